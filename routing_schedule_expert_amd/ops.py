"""Python binding of the C ABI in include/moe.h (ctypes; argument marshalling only).

Every function has the name of its C entry point and takes torch tensors for
the device buffers; the stream defaults to torch's current stream on the
tensors' device.  Each call returns after the launch (asynchronous) and raises
``MoeError`` if the library returns a negative code.  Every step of the layer
runs in the HIP library; if ``libmoe.so`` is missing or a device pointer is not
a CUDA(HIP) tensor, the call fails loudly - there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOSPC, MOE_EUNSUPPORTED, MOE_EHIP = 0, -1, -2, -3, -4
(MOE_OP_SCHEDULE, MOE_OP_DISPATCH, MOE_OP_EXPERT_FFN, MOE_OP_COMBINE, MOE_OP_LAYER_FWD, MOE_OP_LAYER_BWD,
 MOE_OP_LAYER_FWD_SHARED, MOE_OP_LAYER_BWD_MX) = range(8)
MOE_PERSISTENT = 1
MOE_WS_INVALID_IDS, MOE_WS_BARRIER_STATUS = 0, 1
(MOE_WS_MX_DHU, MOE_WS_MX_DO_Q, MOE_WS_MX_DO_S, MOE_WS_MX_DHU_Q, MOE_WS_MX_DHU_S, MOE_WS_MX_DOWT_Q, MOE_WS_MX_DOWT_S,
 MOE_WS_MX_AT_Q, MOE_WS_MX_AT_S, MOE_WS_MX_XDT_Q, MOE_WS_MX_XDT_S, MOE_WS_MX_DHUT_Q, MOE_WS_MX_DHUT_S) = range(2, 15)
MOE_WS_SINGLE_ROUTE = 15

EXPORTED = (
    "moe_strerror", "moe_capacity_rows", "moe_workspace_bytes", "moe_workspace_field", "moe_schedule",
    "moe_dispatch",
    "moe_expert_ffn", "moe_combine", "moe_layer_fwd", "moe_layer_bwd", "moe_trace_enable", "moe_trace_read",
    "moe_quantize_mx", "moe_quantize_mx_t",
    "moe_layer_fwd_mx", "moe_layer_bwd_mx",
    "moe_ring_capacity_rows", "moe_ring_workspace_bytes", "moe_layer_fwd_ring", "moe_layer_bwd_ring",
    "moe_layer_fwd_shared", "moe_layer_fwd_noalloc",
)
MOE_NOALLOC_SCRATCH_BYTES = 8 << 20


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code


class moe_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("P", "Np", "K", "E", "L", "expert_base", "pad_rows", "sched_threads", "H", "I", "num_batches")]


def make_desc(P, Np, K, E, L=None, expert_base=0, pad_rows=256, sched_threads=1024, H=0, I=0, num_batches=1):
    if L is None:
        L = E // P
    return moe_desc(P, Np, K, E, L, expert_base, pad_rows, sched_threads, H, I, num_batches)


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree HIP library (fails loudly when it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with routing_schedule_expert_amd/build.py "
                          "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P, D = ctypes.c_void_p, ctypes.POINTER(moe_desc)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_capacity_rows": (i64, [D]),
        "moe_workspace_bytes": (i64, [D, ctypes.c_int]),
        "moe_workspace_field": (i64, [D, ctypes.c_int, ctypes.c_int]),
        "moe_schedule": (ctypes.c_int, [D, P, P, P, P, P, P, sz, P]),
        "moe_dispatch": (ctypes.c_int, [D, P, P, P, P, P]),
        "moe_expert_ffn": (ctypes.c_int, [D, P, P, P, P, P, P, P, i32, P, sz, P]),
        "moe_combine": (ctypes.c_int, [D, P, P, P, P, P]),
        "moe_layer_fwd": (ctypes.c_int, [D] + [P] * 14 + [i32, i32, P, sz, P]),
        "moe_layer_fwd_noalloc": (ctypes.c_int, [D] + [P] * 14 + [i32, i32, P, P]),
        "moe_quantize_mx": (ctypes.c_int, [P, i64, i32, P, P, P]),
        "moe_quantize_mx_t": (ctypes.c_int, [P, i64, i32, i32, P, P, P]),
        "moe_layer_fwd_mx": (ctypes.c_int, [D] + [P] * 19 + [sz, P]),
        "moe_layer_bwd_mx": (ctypes.c_int, [D] + [P] * 18 + [sz, P]),
        "moe_layer_bwd": (ctypes.c_int, [D] + [P] * 16 + [sz, P]),
        "moe_layer_fwd_shared": (ctypes.c_int, [D, i32] + [P] * 19 + [sz, P]),
        "moe_ring_capacity_rows": (i64, [D, i32]),
        "moe_ring_workspace_bytes": (i64, [D, i32, i32, ctypes.c_int]),
        "moe_layer_fwd_ring": (ctypes.c_int, [D, i32, i32] + [P] * 14 + [sz, P]),
        "moe_layer_bwd_ring": (ctypes.c_int, [D, i32, i32, i32] + [P] * 15 + [sz, P]),
        "moe_trace_enable": (ctypes.c_int, [ctypes.c_int]),
        "moe_trace_read": (ctypes.c_int, [P, P, ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().moe_strerror(code).decode()


def _check(rc: int, where: str) -> int:
    if rc != MOE_OK:
        raise MoeError(rc, where)
    return rc


def _dev(t):
    """Device pointer of a CUDA(HIP) tensor, or NULL for None."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("device buffers must be CUDA (HIP) torch tensors")
    if not t.is_contiguous():
        raise ValueError("device buffers must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, ref: torch.Tensor):
    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    return ctypes.c_void_p(stream.cuda_stream)


def capacity_rows(d: moe_desc) -> int:
    n = load().moe_capacity_rows(ctypes.byref(d))
    if n < 0:
        raise MoeError(MOE_EINVAL, "moe_capacity_rows")
    return int(n)


def workspace_bytes(d: moe_desc, op: int) -> int:
    n = load().moe_workspace_bytes(ctypes.byref(d), op)
    if n < 0:
        raise MoeError(MOE_EINVAL, "moe_workspace_bytes")
    return int(n)


def workspace_field(d: moe_desc, op: int, field: int) -> int:
    """Byte offset of a status word (MOE_WS_*) in op's workspace; -1 if op has none."""
    return int(load().moe_workspace_field(ctypes.byref(d), op, field))


def read_ws_words(ws: torch.Tensor, offset: int, n: int = 1) -> list:
    """The n int32 words at byte `offset` of a workspace tensor (synchronises
    the tensor's stream by copying to the host)."""
    if offset < 0:
        raise ValueError("no such workspace field")
    return [int(v) for v in ws[offset:offset + 4 * n].cpu().view(torch.int32).tolist()]


def moe_schedule(d, routes, counts, seg_off, phi, route_row, ws, stream=None):
    rc = load().moe_schedule(ctypes.byref(d), _dev(routes), _dev(counts), _dev(seg_off), _dev(phi), _dev(route_row),
                             _dev(ws), ws.numel() * ws.element_size(), _stream(stream, routes))
    return _check(rc, "moe_schedule")


def moe_dispatch(d, X, phi, seg_off, Xd, stream=None):
    rc = load().moe_dispatch(ctypes.byref(d), _dev(X), _dev(phi), _dev(seg_off), _dev(Xd), _stream(stream, X))
    return _check(rc, "moe_dispatch")


def moe_expert_ffn(d, Xd, W13, W2, seg_off, HU, A, Y, chunk_rows=0, ws=None, stream=None):
    rc = load().moe_expert_ffn(ctypes.byref(d), _dev(Xd), _dev(W13), _dev(W2), _dev(seg_off), _dev(HU), _dev(A),
                               _dev(Y), chunk_rows, _dev(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream, Xd))
    return _check(rc, "moe_expert_ffn")


def moe_combine(d, Y, route_row, w, out, stream=None):
    rc = load().moe_combine(ctypes.byref(d), _dev(Y), _dev(route_row), _dev(w), _dev(out), _stream(stream, Y))
    return _check(rc, "moe_combine")


def moe_layer_fwd(d, routes, w, X, W13, W2, counts, seg_off, phi, route_row, Xd, HU, A, Y, out, flags=0,
                  chunk_rows=0, ws=None, stream=None):
    rc = load().moe_layer_fwd(ctypes.byref(d), _dev(routes), _dev(w), _dev(X), _dev(W13), _dev(W2), _dev(counts),
                              _dev(seg_off), _dev(phi), _dev(route_row), _dev(Xd), _dev(HU), _dev(A), _dev(Y),
                              _dev(out), flags, chunk_rows, _dev(ws), ws.numel() * ws.element_size(),
                              _stream(stream, X))
    return _check(rc, "moe_layer_fwd")


def moe_layer_fwd_noalloc(d, routes, w, X, W13, W2, counts, seg_off, phi, route_row, Xd, HU, A, Y, out, flags=0,
                          chunk_rows=0, status=None, stream=None):
    rc = load().moe_layer_fwd_noalloc(ctypes.byref(d), _dev(routes), _dev(w), _dev(X), _dev(W13), _dev(W2),
                                      _dev(counts), _dev(seg_off), _dev(phi), _dev(route_row), _dev(Xd), _dev(HU),
                                      _dev(A), _dev(Y), _dev(out), flags, chunk_rows, _dev(status),
                                      _stream(stream, X))
    return _check(rc, "moe_layer_fwd_noalloc")


def moe_layer_bwd(d, dOut, routes, w, phi, route_row, seg_off, Xd, HU, A, W13, W2, dX, dW13, dW2, dw, ws,
                  stream=None):
    rc = load().moe_layer_bwd(ctypes.byref(d), _dev(dOut), _dev(routes), _dev(w), _dev(phi), _dev(route_row),
                              _dev(seg_off), _dev(Xd), _dev(HU), _dev(A), _dev(W13), _dev(W2), _dev(dX), _dev(dW13),
                              _dev(dW2), _dev(dw), _dev(ws), ws.numel() * ws.element_size(), _stream(stream, dOut))
    return _check(rc, "moe_layer_bwd")


def moe_trace_enable(max_records: int) -> None:
    _check(load().moe_trace_enable(max_records), "moe_trace_enable")


def moe_trace_read(max_records: int = 4096):
    """[(kernel name, ms)] of the recorded launches (synchronise first)."""
    names = ctypes.create_string_buffer(32 * max_records)
    ms = (ctypes.c_float * max_records)()
    n = load().moe_trace_read(names, ms, max_records)
    return [(names.raw[32 * i:32 * i + 32].split(b"\0", 1)[0].decode(), float(ms[i])) for i in range(n)]


# ---------------------------------------------------------------------------
# Buffer helpers (device memory via torch; no arithmetic).
# ---------------------------------------------------------------------------

@dataclass
class FwdBuffers:
    counts: torch.Tensor
    seg_off: torch.Tensor
    phi: torch.Tensor
    route_row: torch.Tensor
    Xd: torch.Tensor | None
    HU: torch.Tensor | None
    A: torch.Tensor
    Y: torch.Tensor
    out: torch.Tensor
    ws: torch.Tensor


def alloc_fwd(d: moe_desc, device, save_hu: bool = True, save_xd: bool = True) -> FwdBuffers:
    """Forward buffers.  save_xd=False leaves Xd out: moe_layer_fwd then pulls
    the gate/up rows straight from X (the dispatch fused into the GEMM loads)."""
    cap = capacity_rows(d)
    i32, bf = torch.int32, torch.bfloat16
    return FwdBuffers(
        counts=torch.empty((d.L, d.P), dtype=i32, device=device),
        seg_off=torch.empty(d.L + 1, dtype=i32, device=device),
        phi=torch.empty((cap, 2), dtype=i32, device=device),
        route_row=torch.empty((d.P, d.Np, d.K), dtype=i32, device=device),
        Xd=torch.empty((cap, d.H), dtype=bf, device=device) if save_xd else None,
        HU=torch.empty((cap, 2 * d.I), dtype=bf, device=device) if save_hu else None,
        A=torch.empty((cap, d.I), dtype=bf, device=device),
        Y=torch.empty((cap, d.H), dtype=bf, device=device),
        out=torch.empty((d.P, d.Np, d.H), dtype=bf, device=device),
        ws=torch.empty(max(workspace_bytes(d, MOE_OP_LAYER_FWD), 256), dtype=torch.uint8, device=device),
    )


def layer_fwd(d, routes, w, X, W13, W2, bufs: FwdBuffers, flags=0, chunk_rows=0, stream=None):
    return moe_layer_fwd(d, routes, w, X, W13, W2, bufs.counts, bufs.seg_off, bufs.phi, bufs.route_row, bufs.Xd,
                         bufs.HU, bufs.A, bufs.Y, bufs.out, flags, chunk_rows, bufs.ws, stream)


# ---------------------------------------------------------------------------
# MXFP8 routed experts.
# ---------------------------------------------------------------------------

def moe_quantize_mx(src, q, scales, stream=None):
    """Row-wise MX quantization of a bf16 tensor [..., K] into codes (uint8,
    same shape) and scale bytes (uint8 [..., K/32])."""
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    rc = load().moe_quantize_mx(_dev(src), rows, K, _dev(q), _dev(scales), _stream(stream, src))
    return _check(rc, "moe_quantize_mx")


def quantize_mx(src, stream=None):
    """Allocate and fill (codes, scales) for a bf16 tensor [..., K]."""
    q = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
    s = torch.empty(src.shape[:-1] + (src.shape[-1] // 32,), dtype=torch.uint8, device=src.device)
    moe_quantize_mx(src, q, s, stream)
    return q, s


def moe_quantize_mx_t(src, q, scales, stream=None):
    """MX quantization of the columns of bf16 [..., R, C] along R into codes
    uint8 [..., C, R] and scale bytes uint8 [..., C, R/32]."""
    R, C = src.shape[-2], src.shape[-1]
    batch = src.numel() // (R * C) if R * C else 0
    rc = load().moe_quantize_mx_t(_dev(src), batch, R, C, _dev(q), _dev(scales), _stream(stream, src))
    return _check(rc, "moe_quantize_mx_t")


def quantize_mx_t(src, stream=None):
    """Allocate and fill (codes, scales) of src's columns along its rows."""
    R, C = src.shape[-2], src.shape[-1]
    q = torch.empty(src.shape[:-2] + (C, R), dtype=torch.uint8, device=src.device)
    s = torch.empty(src.shape[:-2] + (C, R // 32), dtype=torch.uint8, device=src.device)
    moe_quantize_mx_t(src, q, s, stream)
    return q, s


def moe_layer_fwd_mx(d, routes, w, X, W13q, W13s, W2q, W2s, counts, seg_off, phi, route_row, Xq, Xs, Aq, As, HU, Y,
                     out, ws, stream=None):
    rc = load().moe_layer_fwd_mx(ctypes.byref(d), _dev(routes), _dev(w), _dev(X), _dev(W13q), _dev(W13s), _dev(W2q),
                                 _dev(W2s), _dev(counts), _dev(seg_off), _dev(phi), _dev(route_row), _dev(Xq),
                                 _dev(Xs), _dev(Aq), _dev(As), _dev(HU), _dev(Y), _dev(out), _dev(ws),
                                 ws.numel() * ws.element_size(), _stream(stream, X))
    return _check(rc, "moe_layer_fwd_mx")


def moe_layer_bwd_mx(d, dOut, w, X, phi, route_row, seg_off, HU, Aq, As, W13tq, W13ts, W2tq, W2ts, dX, dW13, dW2, dw,
                     ws, stream=None):
    rc = load().moe_layer_bwd_mx(ctypes.byref(d), _dev(dOut), _dev(w), _dev(X), _dev(phi), _dev(route_row),
                                 _dev(seg_off), _dev(HU), _dev(Aq), _dev(As), _dev(W13tq), _dev(W13ts), _dev(W2tq),
                                 _dev(W2ts), _dev(dX), _dev(dW13), _dev(dW2), _dev(dw), _dev(ws),
                                 ws.numel() * ws.element_size(), _stream(stream, dOut))
    return _check(rc, "moe_layer_bwd_mx")


@dataclass
class MxFwdBuffers:
    counts: torch.Tensor
    seg_off: torch.Tensor
    phi: torch.Tensor
    route_row: torch.Tensor
    Xq: torch.Tensor
    Xs: torch.Tensor
    Aq: torch.Tensor
    As: torch.Tensor
    HU: torch.Tensor | None
    Y: torch.Tensor
    out: torch.Tensor
    ws: torch.Tensor


def alloc_fwd_mx(d: moe_desc, device, save_hu: bool = False) -> MxFwdBuffers:
    """MX forward buffers; save_hu keeps h and u (bf16) for moe_layer_bwd_mx."""
    cap = capacity_rows(d)
    i32, u8 = torch.int32, torch.uint8
    ntok = d.P * d.Np
    return MxFwdBuffers(
        counts=torch.empty((d.L, d.P), dtype=i32, device=device),
        seg_off=torch.empty(d.L + 1, dtype=i32, device=device),
        phi=torch.empty((cap, 2), dtype=i32, device=device),
        route_row=torch.empty((d.P, d.Np, d.K), dtype=i32, device=device),
        Xq=torch.empty((d.P, d.Np, d.H), dtype=u8, device=device),
        Xs=torch.empty((d.P, d.Np, d.H // 32), dtype=u8, device=device),
        Aq=torch.empty((cap, d.I), dtype=u8, device=device),
        As=torch.empty((cap, d.I // 32), dtype=u8, device=device),
        HU=torch.empty((cap, 2 * d.I), dtype=torch.bfloat16, device=device) if save_hu else None,
        Y=torch.empty((cap, d.H), dtype=torch.bfloat16, device=device),
        out=torch.empty((d.P, d.Np, d.H), dtype=torch.bfloat16, device=device),
        ws=torch.empty(max(workspace_bytes(d, MOE_OP_LAYER_FWD), 256), dtype=torch.uint8, device=device),
    )


def layer_fwd_mx(d, routes, w, X, W13q, W13s, W2q, W2s, bufs: MxFwdBuffers, stream=None):
    return moe_layer_fwd_mx(d, routes, w, X, W13q, W13s, W2q, W2s, bufs.counts, bufs.seg_off, bufs.phi,
                            bufs.route_row, bufs.Xq, bufs.Xs, bufs.Aq, bufs.As, bufs.HU, bufs.Y, bufs.out, bufs.ws,
                            stream)


@dataclass
class MxBwdGrads:
    dX: torch.Tensor
    dW13: torch.Tensor
    dW2: torch.Tensor
    dw: torch.Tensor
    ws: torch.Tensor


def alloc_bwd_mx(d: moe_desc, device) -> MxBwdGrads:
    return MxBwdGrads(
        dX=torch.empty((d.P, d.Np, d.H), dtype=torch.bfloat16, device=device),
        dW13=torch.empty((d.L, 2 * d.I, d.H), dtype=torch.float32, device=device),
        dW2=torch.empty((d.L, d.H, d.I), dtype=torch.float32, device=device),
        dw=torch.empty((d.P, d.Np, d.K), dtype=torch.float32, device=device),
        ws=torch.empty(workspace_bytes(d, MOE_OP_LAYER_BWD_MX), dtype=torch.uint8, device=device),
    )


def mx_bwd_views(d: moe_desc, ws: torch.Tensor) -> dict:
    """Views of moe_layer_bwd_mx's workspace buffers (the MOE_WS_MX_* fields):
    dHU bf16 [cap][2I]; row codes / scales (DO, DHU) [cap][C] / [cap][C/32];
    the column codes (DOWT, AT, XDT, DHUT) as flat (codes, scales) byte
    tensors, segment-major (mx_expert_block cuts one expert's block out)."""
    cap = capacity_rows(d)
    H, I2 = d.H, 2 * d.I

    def at(field, nbytes):
        off = workspace_field(d, MOE_OP_LAYER_BWD_MX, field)
        return ws[off:off + nbytes]

    v = {"dHU": at(MOE_WS_MX_DHU, cap * I2 * 2).view(torch.bfloat16).view(cap, I2)}
    for nm, f, C in (("DO", MOE_WS_MX_DO_Q, H), ("DHU", MOE_WS_MX_DHU_Q, I2)):
        v[nm] = (at(f, cap * C).view(cap, C), at(f + 1, cap * C // 32).view(cap, C // 32))
    for nm, f, C in (("DOWT", MOE_WS_MX_DOWT_Q, H), ("AT", MOE_WS_MX_AT_Q, d.I), ("XDT", MOE_WS_MX_XDT_Q, H),
                     ("DHUT", MOE_WS_MX_DHUT_Q, I2)):
        v[nm] = (at(f, cap * C), at(f + 1, cap * C // 32), C)
    return v


def mx_expert_block(view, S: int, n: int):
    """(codes [C][n], scales [C][n/32]) of the expert whose rows are [S, S+n)
    in a segment-major column-code view of mx_bwd_views."""
    q, s, C = view
    return q[C * S:C * (S + n)].view(C, n), s[C * S // 32:C * (S + n) // 32].view(C, n // 32)


def layer_bwd_mx(d, dOut, w, X, fwd: MxFwdBuffers, W13t, W2t, g: MxBwdGrads, stream=None):
    """moe_layer_bwd_mx on a forward's buffers; W13t / W2t are the (codes,
    scales) of quantize_mx_t(W13) and quantize_mx_t(W2)."""
    return moe_layer_bwd_mx(d, dOut, w, X, fwd.phi, fwd.route_row, fwd.seg_off, fwd.HU, fwd.Aq, fwd.As, W13t[0],
                            W13t[1], W2t[0], W2t[1], g.dX, g.dW13, g.dW2, g.dw, g.ws, stream)


# ---------------------------------------------------------------------------
# Macrobatch ring.
# ---------------------------------------------------------------------------

def ring_capacity_rows(d: moe_desc, mb_tokens: int) -> int:
    n = load().moe_ring_capacity_rows(ctypes.byref(d), mb_tokens)
    if n < 0:
        raise MoeError(MOE_EINVAL, "moe_ring_capacity_rows")
    return int(n)


def ring_workspace_bytes(d: moe_desc, mb_tokens: int, op: int, wgrad_group: int = 1) -> int:
    n = load().moe_ring_workspace_bytes(ctypes.byref(d), mb_tokens, wgrad_group, op)
    if n < 0:
        raise MoeError(MOE_EINVAL, "moe_ring_workspace_bytes")
    return int(n)


def moe_layer_fwd_ring(d, mb_tokens, ring_slots, routes, w, X, W13, W2, counts, seg_off, phi, route_row, HU, A, Y,
                       out, ws, stream=None):
    rc = load().moe_layer_fwd_ring(ctypes.byref(d), mb_tokens, ring_slots, _dev(routes), _dev(w), _dev(X), _dev(W13),
                                   _dev(W2), _dev(counts), _dev(seg_off), _dev(phi), _dev(route_row), _dev(HU),
                                   _dev(A), _dev(Y), _dev(out), _dev(ws), ws.numel() * ws.element_size(),
                                   _stream(stream, X))
    return _check(rc, "moe_layer_fwd_ring")


def moe_layer_bwd_ring(d, mb_tokens, ring_slots, dOut, w, X, W13, W2, phi, route_row, seg_off, HU, A, dX, dW13, dW2,
                       dw, ws, stream=None, wgrad_group=1):
    rc = load().moe_layer_bwd_ring(ctypes.byref(d), mb_tokens, ring_slots, wgrad_group, _dev(dOut), _dev(w), _dev(X),
                                   _dev(W13),
                                   _dev(W2), _dev(phi), _dev(route_row), _dev(seg_off), _dev(HU), _dev(A), _dev(dX),
                                   _dev(dW13), _dev(dW2), _dev(dw), _dev(ws), ws.numel() * ws.element_size(),
                                   _stream(stream, dOut))
    return _check(rc, "moe_layer_bwd_ring")


@dataclass
class RingBuffers:
    mb_tokens: int
    slots: int
    counts: torch.Tensor     # [M][L][P]
    seg_off: torch.Tensor    # [M][L+1]
    phi: torch.Tensor        # [M][capm][2]
    route_row: torch.Tensor  # [P][Np][K]
    HU: torch.Tensor         # [slots][capm][2I]
    A: torch.Tensor          # [slots][capm][I]
    Y: torch.Tensor          # [capm][H]
    out: torch.Tensor
    ws: torch.Tensor


def alloc_ring(d: moe_desc, mb_tokens: int, slots: int, device) -> RingBuffers:
    capm = ring_capacity_rows(d, mb_tokens)
    M = d.Np // mb_tokens
    i32, bf = torch.int32, torch.bfloat16
    return RingBuffers(
        mb_tokens=mb_tokens, slots=slots,
        counts=torch.empty((M, d.L, d.P), dtype=i32, device=device),
        seg_off=torch.empty((M, d.L + 1), dtype=i32, device=device),
        phi=torch.empty((M, capm, 2), dtype=i32, device=device),
        route_row=torch.empty((d.P, d.Np, d.K), dtype=i32, device=device),
        HU=torch.empty((slots, capm, 2 * d.I), dtype=bf, device=device),
        A=torch.empty((slots, capm, d.I), dtype=bf, device=device),
        Y=torch.empty((capm, d.H), dtype=bf, device=device),
        out=torch.empty((d.P, d.Np, d.H), dtype=bf, device=device),
        ws=torch.empty(max(ring_workspace_bytes(d, mb_tokens, MOE_OP_LAYER_FWD), 256), dtype=torch.uint8,
                       device=device),
    )


def layer_fwd_ring(d, routes, w, X, W13, W2, r: RingBuffers, stream=None):
    return moe_layer_fwd_ring(d, r.mb_tokens, r.slots, routes, w, X, W13, W2, r.counts, r.seg_off, r.phi,
                              r.route_row, r.HU, r.A, r.Y, r.out, r.ws, stream)


# ---------------------------------------------------------------------------
# Shared expert.
# ---------------------------------------------------------------------------

def moe_layer_fwd_shared(d, Is, routes, w, X, W13, W2, W13s, W2s, counts, seg_off, phi, route_row, HU, A, Y, HUs, As,
                         Ys, out, ws, stream=None):
    rc = load().moe_layer_fwd_shared(ctypes.byref(d), Is, _dev(routes), _dev(w), _dev(X), _dev(W13), _dev(W2),
                                     _dev(W13s), _dev(W2s), _dev(counts), _dev(seg_off), _dev(phi), _dev(route_row),
                                     _dev(HU), _dev(A), _dev(Y), _dev(HUs), _dev(As), _dev(Ys), _dev(out), _dev(ws),
                                     ws.numel() * ws.element_size(), _stream(stream, X))
    return _check(rc, "moe_layer_fwd_shared")


@dataclass
class SharedBuffers:
    Is: int
    HUs: torch.Tensor | None
    As: torch.Tensor
    Ys: torch.Tensor
    ws: torch.Tensor


def alloc_shared(d: moe_desc, Is: int, device, save_hu: bool = False) -> SharedBuffers:
    ntokp = (d.P * d.Np + 255) // 256 * 256
    bf = torch.bfloat16
    return SharedBuffers(
        Is=Is,
        HUs=torch.empty((ntokp, 2 * Is), dtype=bf, device=device) if save_hu else None,
        As=torch.empty((ntokp, Is), dtype=bf, device=device),
        Ys=torch.empty((ntokp, d.H), dtype=bf, device=device),
        ws=torch.empty(workspace_bytes(d, MOE_OP_LAYER_FWD_SHARED), dtype=torch.uint8, device=device),
    )


def layer_fwd_shared(d, routes, w, X, W13, W2, W13s, W2s, bufs: FwdBuffers, sh: SharedBuffers, stream=None):
    """Forward with a shared expert; bufs.Xd is not used (fused dispatch)."""
    return moe_layer_fwd_shared(d, sh.Is, routes, w, X, W13, W2, W13s, W2s, bufs.counts, bufs.seg_off, bufs.phi,
                                bufs.route_row, bufs.HU, bufs.A, bufs.Y, sh.HUs, sh.As, sh.Ys, bufs.out, sh.ws, stream)
