"""moe_layer_fwd_noalloc (the layer forward for callers that cannot allocate:
its workspace is a static device array of the library) against
moe_layer_fwd with a caller-allocated workspace: every output bitwise equal,
on two calls in a row, the second with a smaller input, on the multi-launch
and persistent paths; the status words it reports; the size limit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs, ops
from tests.helpers import dev, fused_y_rows, on_dev_mask, up, up_bf16

pytestmark = pytest.mark.gpu

FIELDS = ("counts", "seg_off", "phi", "route_row", "Xd", "HU", "A", "Y", "out")


def make(seed, P, Np, E, K, L, H, I, routing):
    h = inputs.make_layer_inputs(seed, P, Np, E, K, L, H, I, routing=routing, x_std=1.0)
    d = ops.make_desc(P, Np, K, E, L, H=H, I=I)
    return h, d, up(h["routes"]), up(h["w"]), up_bf16(h["X"]), up_bf16(h["W13"]), up_bf16(h["W2"])


def run_both(h, d, routes, w, X, W13, W2, flags, save_xd):
    ref = ops.alloc_fwd(d, dev(), save_xd=save_xd)
    ops.layer_fwd(d, routes, w, X, W13, W2, ref, flags=flags)
    got = ops.alloc_fwd(d, dev(), save_xd=save_xd)
    status = torch.full((2,), -9, dtype=torch.int32, device=dev())
    ops.moe_layer_fwd_noalloc(d, routes, w, X, W13, W2, got.counts, got.seg_off, got.phi, got.route_row, got.Xd,
                              got.HU, got.A, got.Y, got.out, flags=flags, status=status)
    torch.cuda.synchronize()
    npad = int(ref.seg_off[-1])
    for name in FIELDS:
        a, b = getattr(ref, name), getattr(got, name)
        if a is None:
            assert b is None
            continue
        if name in ("phi", "Xd", "HU", "A", "Y"):
            a, b = a[:npad], b[:npad]
        if name == "Y" and not flags:  # rows of one-route tokens go straight to out
            yw = on_dev_mask(fused_y_rows(h["routes"], d.L, d.expert_base, ref.phi[:npad].cpu().numpy()))
            a, b = a[yw], b[yw]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name} differs (flags={flags})"
    st = status.cpu().tolist()
    assert st == [oracle.invalid_ids(h["routes"], d.E), 0], st
    return npad


@pytest.mark.parametrize("flags", [0, ops.MOE_PERSISTENT])
def test_noalloc_matches_layer_fwd_twice_shrinking(flags):
    print(f"[noalloc] flags={flags}: larger call", flush=True)
    big = make(21, 8, 1500, 64, 6, 8, 1024, 512, "zipf")
    big_rt = big[0]["routes"].copy()
    big_rt[1, ::7, 2] = -1  # dropped slots reach the invalid-id count
    big[0]["routes"] = big_rt
    big = (big[0], big[1], up(big_rt)) + big[3:]
    n1 = run_both(*big, flags=flags, save_xd=True)
    print(f"[noalloc] flags={flags}: smaller call", flush=True)
    small = make(22, 2, 256, 8, 2, 4, 256, 128, "topk")
    n2 = run_both(*small, flags=flags, save_xd=False)
    assert n2 < n1


def test_noalloc_rejects_workspace_past_the_array():
    d = ops.make_desc(8, 7168 * 16, 8, 384, 48, H=7168, I=2048)
    assert ops.workspace_bytes(d, ops.MOE_OP_LAYER_FWD) > ops.MOE_NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.int32, device=dev())
    p = ctypes.c_void_p(t.data_ptr())
    rc = ops.load().moe_layer_fwd_noalloc(ctypes.byref(d), *([p] * 14), 0, 0, None,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == ops.MOE_ENOSPC
