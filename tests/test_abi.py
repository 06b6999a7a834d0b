"""The C-ABI library on the host (no GPU needed).

The library must load, export every function include/moe.h declares, size its
buffers as documented, and reject bad arguments with the documented codes
before anything is launched (checked with NULL or host-only arguments, so no
device code ever runs here).
"""
import ctypes
import re
import os

import pytest

from routing_schedule_expert_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = ops.load()
    names = declared_functions()
    assert set(names) == set(ops.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_strerror():
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(ops.strerror(code), str) and ops.strerror(code)


def kimi():
    return ops.make_desc(8, 7168, 8, 384, 48, H=7168, I=2048)


def test_capacity_and_workspace_sizes():
    d = kimi()
    assert ops.capacity_rows(d) == 8 * 7168 * 8 + 48 * 255 == 470992
    assert ops.workspace_bytes(d, ops.MOE_OP_DISPATCH) == 0
    assert ops.workspace_bytes(d, ops.MOE_OP_SCHEDULE) > 0
    d64 = kimi()
    d64.num_batches = 64
    routes = 8 * 7168 * 8
    # per-chunk counters (at least one int per batch, partition and expert) and
    # one byte per route for the scatter's second read of the local ids
    assert ops.workspace_bytes(d, ops.MOE_OP_SCHEDULE) >= 8 * 48 * 4 + routes
    assert ops.workspace_bytes(d64, ops.MOE_OP_SCHEDULE) >= 64 * (8 * 48 * 4 + routes)
    # more than 255 local experts: no byte copy (the scatter reads the ids again),
    # so one more local expert takes less workspace
    w255 = ops.workspace_bytes(ops.make_desc(8, 7168, 8, 2048, 255), ops.MOE_OP_SCHEDULE)
    w256 = ops.workspace_bytes(ops.make_desc(8, 7168, 8, 2048, 256), ops.MOE_OP_SCHEDULE)
    assert 0 < w256 < w255 and w255 >= routes
    cap = ops.capacity_rows(d)
    assert ops.workspace_bytes(d, ops.MOE_OP_LAYER_BWD) >= cap * (7168 * 2 + 4096) * 2


@pytest.mark.parametrize("field,value", [
    ("P", 0), ("Np", 0), ("K", 0), ("E", 0), ("L", 0), ("pad_rows", 0), ("sched_threads", 0),
    ("num_batches", 0), ("expert_base", -1), ("expert_base", 337),
])
def test_invalid_descriptor(field, value):
    d = kimi()
    setattr(d, field, value)
    assert ops.load().moe_capacity_rows(ctypes.byref(d)) == -1
    assert ops.load().moe_workspace_bytes(ctypes.byref(d), ops.MOE_OP_SCHEDULE) == -1


def test_unsupported_shapes():
    lib = ops.load()
    for H, I, pad in ((7000, 2048, 256), (7168, 2000, 256), (7168, 2048, 128)):
        d = ops.make_desc(8, 7168, 8, 384, 48, pad_rows=pad, H=H, I=I)
        assert lib.moe_workspace_bytes(ctypes.byref(d), ops.MOE_OP_EXPERT_FFN) == -1
        rc = lib.moe_expert_ffn(ctypes.byref(d), *([None] * 7), 0, None, 0, None)
        assert rc == ops.MOE_EUNSUPPORTED
    d = ops.make_desc(8, 7168, 8, 4096 * 8, 4096)  # L*P beyond the supported table size
    assert lib.moe_capacity_rows(ctypes.byref(d)) == -1
    # GEMM tiles are numbered with 32-bit integers: a shape with ~4e10 weight-
    # gradient tiles is refused (its weights alone would be petabytes)
    big = ops.make_desc(8, 7168, 8, 384, 48, H=1 << 22, I=1 << 22)
    assert lib.moe_workspace_bytes(ctypes.byref(big), ops.MOE_OP_LAYER_BWD) == -1
    assert lib.moe_expert_ffn(ctypes.byref(big), *([None] * 7), 0, None, 0, None) == ops.MOE_EUNSUPPORTED
    ok = ops.make_desc(8, 7168, 8, 384, 48, H=1 << 15, I=1 << 14)
    assert lib.moe_workspace_bytes(ctypes.byref(ok), ops.MOE_OP_LAYER_BWD) > 0


def test_null_arguments_rejected_before_launch():
    lib = ops.load()
    d = kimi()
    assert lib.moe_schedule(None, *([None] * 6), 0, None) == ops.MOE_EINVAL
    assert lib.moe_schedule(ctypes.byref(d), *([None] * 6), 0, None) == ops.MOE_EINVAL
    assert lib.moe_dispatch(ctypes.byref(d), *([None] * 4), None) == ops.MOE_EINVAL
    assert lib.moe_combine(ctypes.byref(d), *([None] * 4), None) == ops.MOE_EINVAL
    assert lib.moe_expert_ffn(ctypes.byref(d), *([None] * 7), 0, None, 0, None) == ops.MOE_EINVAL
    assert lib.moe_layer_fwd(ctypes.byref(d), *([None] * 14), 0, 0, None, 0, None) == ops.MOE_EINVAL
    assert lib.moe_layer_bwd(ctypes.byref(d), *([None] * 16), 0, None) == ops.MOE_EINVAL


def _fake(addr):
    # aligned, non-NULL host addresses: every call below fails its host-side
    # checks before it could launch anything that dereferences them
    return ctypes.c_void_p(addr)


def test_small_workspace_and_misalignment():
    lib = ops.load()
    d = kimi()
    p = [_fake(0x10000 * (i + 1)) for i in range(8)]
    need = lib.moe_workspace_bytes(ctypes.byref(d), ops.MOE_OP_SCHEDULE)
    assert lib.moe_schedule(ctypes.byref(d), *p[:6], need - 1, None) == ops.MOE_ENOSPC
    bad = _fake(0x10004)
    assert lib.moe_schedule(ctypes.byref(d), bad, *p[1:6], need, None) == ops.MOE_EINVAL
    # chunk_rows must be a non-negative multiple of 256
    assert lib.moe_expert_ffn(ctypes.byref(d), *p[:4], None, p[4], p[5], 100, p[6], 256, None) == ops.MOE_EINVAL
    # the forward layer call takes one routing tensor
    d2 = kimi()
    d2.num_batches = 2
    args = p[:5] + p[:4] + [p[4], None, p[5], p[6], p[7]]
    assert lib.moe_layer_fwd(ctypes.byref(d2), *args, 0, 0, p[0], 1 << 30, None) == ops.MOE_EINVAL
    # unknown flag bits
    assert lib.moe_layer_fwd(ctypes.byref(d), *args, 8, 0, p[0], 1 << 30, None) == ops.MOE_EINVAL
    # backward workspace too small
    nbwd = lib.moe_workspace_bytes(ctypes.byref(d), ops.MOE_OP_LAYER_BWD)
    bargs = [p[i % 8] for i in range(16)]
    assert lib.moe_layer_bwd(ctypes.byref(d), *bargs, nbwd - 1, None) == ops.MOE_ENOSPC


def test_fused_dispatch_needs_zero_row():
    # Xd = NULL pulls padding rows from a 32768-element zero row: wider H is refused before any launch
    lib = ops.load()
    d = ops.make_desc(8, 7168, 8, 384, 48, H=32768 + 256, I=2048)
    p = [_fake(0x10000 * (i + 1)) for i in range(8)]
    args = p[:5] + p[:4] + [None, None, p[5], p[6], p[7]]
    ws = lib.moe_workspace_bytes(ctypes.byref(d), ops.MOE_OP_LAYER_FWD)
    assert ws > 0
    assert lib.moe_layer_fwd(ctypes.byref(d), *args, 0, 0, p[0], ws, None) == ops.MOE_EUNSUPPORTED


def test_schedule_lds_limit():
    # 4,096 local experts: the scatter's per-expert LDS tables exceed 160 KiB -> refused before any launch
    lib = ops.load()
    d = ops.make_desc(4, 1024, 8, 4096, 4096)
    ws = lib.moe_workspace_bytes(ctypes.byref(d), ops.MOE_OP_SCHEDULE)
    assert ws > 0
    p = [_fake(0x10000 * (i + 1)) for i in range(6)]
    assert lib.moe_schedule(ctypes.byref(d), *p, ws, None) == ops.MOE_EUNSUPPORTED


def test_mx_arguments_rejected_before_launch():
    lib = ops.load()
    p = [_fake(0x10000 * (i + 1)) for i in range(20)]
    assert lib.moe_quantize_mx(p[0], 4, 48, p[1], p[2], None) == ops.MOE_EINVAL  # K not a multiple of 32
    assert lib.moe_quantize_mx(p[0], -1, 64, p[1], p[2], None) == ops.MOE_EINVAL
    assert lib.moe_quantize_mx(_fake(0x10008), 4, 64, p[1], p[2], None) == ops.MOE_EINVAL  # misaligned
    assert lib.moe_quantize_mx(None, 0, 64, None, None, None) == ops.MOE_OK  # nothing to do
    d = kimi()
    ws = lib.moe_workspace_bytes(ctypes.byref(d), ops.MOE_OP_LAYER_FWD)
    args = p[:19]  # 18 operands and the workspace
    assert lib.moe_layer_fwd_mx(ctypes.byref(d), *args[:5], None, *args[6:], ws, None) == ops.MOE_EINVAL
    assert lib.moe_layer_fwd_mx(ctypes.byref(d), *args[:3], _fake(0x10004), *args[4:], ws, None) == ops.MOE_EINVAL
    assert lib.moe_layer_fwd_mx(ctypes.byref(d), *args, ws - 1, None) == ops.MOE_ENOSPC
    d2 = ops.make_desc(8, 7168, 8, 384, 48, H=65536 + 256, I=2048)  # rows wider than the zero row for padding
    ws2 = lib.moe_workspace_bytes(ctypes.byref(d2), ops.MOE_OP_LAYER_FWD)
    assert lib.moe_layer_fwd_mx(ctypes.byref(d2), *args, ws2, None) == ops.MOE_EUNSUPPORTED
    # HU (operand 15) is optional but must be 16-byte aligned when given
    assert lib.moe_layer_fwd_mx(ctypes.byref(d), *args[:15], _fake(0x10008), *args[16:], ws, None) == ops.MOE_EINVAL


def test_mx_backward_arguments_and_workspace():
    lib = ops.load()
    p = [_fake(0x10000 * (i + 1)) for i in range(20)]
    # column quantization: R a multiple of 32, C of 8, aligned pointers
    assert lib.moe_quantize_mx_t(p[0], 2, 48, 64, p[1], p[2], None) == ops.MOE_EINVAL
    assert lib.moe_quantize_mx_t(p[0], 2, 64, 60, p[1], p[2], None) == ops.MOE_EINVAL
    assert lib.moe_quantize_mx_t(p[0], -1, 64, 64, p[1], p[2], None) == ops.MOE_EINVAL
    assert lib.moe_quantize_mx_t(_fake(0x10008), 1, 64, 64, p[1], p[2], None) == ops.MOE_EINVAL
    assert lib.moe_quantize_mx_t(None, 0, 64, 64, None, None, None) == ops.MOE_OK
    d = kimi()
    cap = ops.capacity_rows(d)
    wm = ops.workspace_bytes(d, ops.MOE_OP_LAYER_BWD_MX)
    H, I = 7168, 2048
    # dXd and dHU (bf16), the row weights and dw partials (fp32), the row
    # codes of dO_d and dHU and the four column-coded operands (C codes per
    # dispatched row); codes plus a scale byte per 32
    need = cap * (2 * H + 4 * I + 4 + 4 * (I // 256)) + cap * (3 * H + 5 * I) * 33 // 32
    assert need <= wm <= need + 16 * 256
    bwd = p[:18]  # 17 operands and the workspace
    assert lib.moe_layer_bwd_mx(ctypes.byref(d), *bwd, wm - 1, None) == ops.MOE_ENOSPC
    for i in range(18):
        assert lib.moe_layer_bwd_mx(ctypes.byref(d), *bwd[:i], None, *bwd[i + 1:], wm, None) == ops.MOE_EINVAL, i
    assert lib.moe_layer_bwd_mx(ctypes.byref(d), _fake(0x10008), *bwd[1:], wm, None) == ops.MOE_EINVAL
    d2 = ops.make_desc(8, 7168, 8, 384, 48, H=7168, I=2048, num_batches=2)
    assert lib.moe_layer_bwd_mx(ctypes.byref(d2), *bwd, wm, None) == ops.MOE_EINVAL


def test_ring_sizes_and_arguments_rejected_before_launch():
    lib = ops.load()
    d = kimi()
    assert ops.ring_capacity_rows(d, 1024) == 8 * 1024 * 8 + 48 * 255
    assert ops.ring_capacity_rows(d, 7168) == ops.capacity_rows(d)
    for bad in (0, -1, 1000, 7169):  # must divide Np
        assert lib.moe_ring_capacity_rows(ctypes.byref(d), bad) == -1
    assert lib.moe_ring_workspace_bytes(ctypes.byref(d), 1024, 1, ops.MOE_OP_SCHEDULE) == -1
    for bad_group in (0, 17):
        assert lib.moe_ring_workspace_bytes(ctypes.byref(d), 1024, bad_group, ops.MOE_OP_LAYER_BWD) == -1
    wf = ops.ring_workspace_bytes(d, 1024, ops.MOE_OP_LAYER_FWD)
    wb = ops.ring_workspace_bytes(d, 1024, ops.MOE_OP_LAYER_BWD)
    # each macrobatch of a weight-gradient group keeps its own rows; 7 macrobatches at most
    w3, w7, w9 = (ops.ring_workspace_bytes(d, 1024, ops.MOE_OP_LAYER_BWD, g) for g in (3, 7, 9))
    assert wb < w3 < w7 == w9
    capm = ops.ring_capacity_rows(d, 1024)
    assert wb >= capm * (7168 * 3 + 2048 * 3) * 2  # per-slot dO_d, dXd, Xd, dHU, replayed HU and A
    p = [_fake(0x10000 * (i + 1)) for i in range(20)]
    fwd = p[:14]  # 13 operands and the workspace
    bwd = p[:15]  # 14 operands and the workspace
    for mb, slots in ((1000, 2), (0, 2), (1024, 0)):
        assert lib.moe_layer_fwd_ring(ctypes.byref(d), mb, slots, *fwd, wf, None) == ops.MOE_EINVAL
        assert lib.moe_layer_bwd_ring(ctypes.byref(d), mb, slots, 1, *bwd, wb, None) == ops.MOE_EINVAL
    assert lib.moe_layer_fwd_ring(ctypes.byref(d), 1024, 2, *fwd[:4], None, *fwd[5:], wf, None) == ops.MOE_EINVAL
    assert lib.moe_layer_fwd_ring(ctypes.byref(d), 1024, 2, *fwd[:9], _fake(0x10004), *fwd[10:], wf,
                                  None) == ops.MOE_EINVAL
    assert lib.moe_layer_fwd_ring(ctypes.byref(d), 1024, 2, *fwd, wf - 1, None) == ops.MOE_ENOSPC
    assert lib.moe_layer_bwd_ring(ctypes.byref(d), 1024, 2, 1, *bwd[:14], None, wb, None) == ops.MOE_EINVAL
    assert lib.moe_layer_bwd_ring(ctypes.byref(d), 1024, 2, 1, *bwd, wb - 1, None) == ops.MOE_ENOSPC
    assert lib.moe_layer_bwd_ring(ctypes.byref(d), 1024, 2, 0, *bwd, 1 << 40, None) == ops.MOE_EINVAL
    assert lib.moe_layer_bwd_ring(ctypes.byref(d), 1024, 2, 3, *bwd, w3 - 1, None) == ops.MOE_ENOSPC
    d2 = ops.make_desc(8, 7168, 8, 384, 48, H=65536 + 256, I=2048)
    assert lib.moe_layer_fwd_ring(ctypes.byref(d2), 1024, 2, *fwd, 1 << 40, None) == ops.MOE_EUNSUPPORTED


def test_trace_read_empty():
    assert ops.moe_trace_read(4) == []


def test_workspace_fields():
    """Status words: the invalid-id counts sit at the start of the schedule's
    workspace (after the 256 barrier bytes in the layer forward), the barrier
    give-up word at byte 8 of the calls that wait across workgroups."""
    d = kimi()
    f = ops.workspace_field
    assert f(d, ops.MOE_OP_SCHEDULE, ops.MOE_WS_INVALID_IDS) == 0
    assert f(d, ops.MOE_OP_LAYER_FWD, ops.MOE_WS_INVALID_IDS) == 256
    assert f(d, ops.MOE_OP_LAYER_FWD_SHARED, ops.MOE_WS_INVALID_IDS) == 256
    assert f(d, ops.MOE_OP_LAYER_FWD, ops.MOE_WS_BARRIER_STATUS) == 8
    assert f(d, ops.MOE_OP_EXPERT_FFN, ops.MOE_WS_BARRIER_STATUS) == 8
    for op, field in ((ops.MOE_OP_SCHEDULE, ops.MOE_WS_BARRIER_STATUS), (ops.MOE_OP_DISPATCH, 0),
                      (ops.MOE_OP_LAYER_BWD, 0), (ops.MOE_OP_LAYER_FWD, 7)):
        assert f(d, op, field) == -1
    for op in (ops.MOE_OP_SCHEDULE, ops.MOE_OP_LAYER_FWD):
        off = f(d, op, ops.MOE_WS_INVALID_IDS)
        assert 0 <= off and off + 4 <= ops.workspace_bytes(d, op)
    # the forward's single-route table: 8 bytes per row of capacity, at the end
    off = f(d, ops.MOE_OP_LAYER_FWD, ops.MOE_WS_SINGLE_ROUTE)
    assert off > 256 and off % 256 == 0
    assert off + 8 * ops.capacity_rows(d) <= ops.workspace_bytes(d, ops.MOE_OP_LAYER_FWD) < off + 8 * ops.capacity_rows(d) + 256
    for op in (ops.MOE_OP_SCHEDULE, ops.MOE_OP_LAYER_FWD_SHARED, ops.MOE_OP_LAYER_BWD):
        assert f(d, op, ops.MOE_WS_SINGLE_ROUTE) == -1
    bad = kimi()
    bad.P = 0
    assert f(bad, ops.MOE_OP_SCHEDULE, ops.MOE_WS_INVALID_IDS) == -1


def test_route_count_bound():
    """Routes per partition up to the 32-bit capacity bound are accepted (the
    schedule indexes its blocks with 64-bit starts), one more is not."""
    lib = ops.load()
    # P = 1, K = 1, L = 1, pad 256: cap = Np + 255 must stay below 2^31 - 256
    ok = ops.make_desc(1, 2**31 - 1024, 1, 2, 1)
    assert lib.moe_capacity_rows(ctypes.byref(ok)) == 2**31 - 1024 + 255
    assert lib.moe_workspace_bytes(ctypes.byref(ok), ops.MOE_OP_SCHEDULE) > 2**31 - 1024
    over = ops.make_desc(1, 2**31 - 511, 1, 2, 1)
    assert lib.moe_capacity_rows(ctypes.byref(over)) == -1
