"""CPU oracle for one GPU's share of the Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library (``routing_schedule_expert_amd``) and never
imports it.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision, built with
gcc); this module marshals numpy arrays, except ``mx_layer_bwd``, which writes
the MXFP8 backward a second time in matrix form (numpy fp64 products on
dequantized operands, per expert segment), fast enough for full experts at
the Kimi shape, and pinned against the C loops.  Every function names the page
and section it follows.

Parity status of each function (what pins it is in ``tests/test_oracle_*.py``):
  schedule, schedule_counting, schedule_rescan  pinned (brute force, closed forms,
                                                  printed read/counter counts,
                                                  stable-argsort special case)
  dispatch                                       pinned (bit copy by definition)
  expert_ffn_rows, layer_fwd_tokens, combine     pinned (dense FFN special case vs
                                                  torch fp64, un-permute special case)
  layer_bwd, bwd_tokens, wgrad_elems             pinned (finite differences, torch
                                                  autograd, the dw identity)
  minibatch_floor                                pinned (the printed 2368)
  invalid_ids                                    pinned (brute force on tiny inputs)
  e4m3_value, e4m3_encode, mx_quantize,          pinned (E4M3 closed form per code, encode-
    mx_quantize_f64, mx_dequantize                 decode identity, ties to even, saturation,
                                                   scale exponent of the block maximum)
  mx_expert_ffn_rows, mx_layer_fwd_tokens        pinned (dot products vs numpy on the
                                                   dequantized operands; token path = rows +
                                                   combine; close to the bf16 FFN)
  mx_weights_t, mx_bwd_tokens, mx_wgrad_elems,   pinned (the C loops and the matrix form agree
    mx_layer_bwd                                   to 1e-12 at tiny shapes; within the format's
                                                   error of the bf16 backward; exact scaling by
                                                   powers of two of dOut; zero dOut, non-local
                                                   tokens)
  shared_ffn_tokens, layer_fwd_tokens_shared     pinned (dense SwiGLU vs torch fp64 with no
                                                   local routes; zero shared weights leave the
                                                   routed output; the routed part stays linear
                                                   in w)
  macrobatch_schedules, ring_walk                pinned (one macrobatch = the whole table;
                                                   every local route in exactly one window;
                                                   closed forms of the reversed ring's
                                                   residency and replay count)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
# MOE_ORACLE_LIB names another build of moe_oracle.c to load instead (the
# sanitizer build of oracle/sanitize.sh); it is used as it is, never rebuilt.
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP) into ``oracle/libmoe_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        lib.orc_capacity_rows.argtypes = [i32, i32, i32, i32, i32]
        lib.orc_capacity_rows.restype = i64
        lib.orc_minibatch_floor.argtypes = [i64] * 5
        lib.orc_minibatch_floor.restype = i64
        sched = [i32, i32, i32, i32, i32, i32, p, p, p, p, i64, p, p]
        lib.orc_schedule.argtypes = sched
        lib.orc_schedule.restype = i64
        lib.orc_schedule_rescan.argtypes = sched
        lib.orc_schedule_rescan.restype = i64
        lib.orc_schedule_counting.argtypes = [i32] * 7 + [p, p, p, p, i64, p, p]
        lib.orc_schedule_counting.restype = i64
        lib.orc_invalid_ids.argtypes = [i64, i32, p]
        lib.orc_invalid_ids.restype = i64
        lib.orc_dispatch.argtypes = [i32, i32, p, p, i64, p]
        lib.orc_dispatch.restype = None
        lib.orc_expert_ffn_rows.argtypes = [i32, i32, i32, p, p, p, p, p, i64, p, p, p]
        lib.orc_expert_ffn_rows.restype = None
        lib.orc_combine_tokens.argtypes = [i32, i32, i32, p, p, p, p, p, i64, p]
        lib.orc_combine_tokens.restype = None
        lib.orc_layer_fwd_tokens.argtypes = [i32, i32, i32, i32, i32, p, p, p, p, p, p, i64, p]
        lib.orc_layer_fwd_tokens.restype = None
        lib.orc_layer_bwd.argtypes = [i64, i32, i32, i32, i32, i32] + [p] * 10
        lib.orc_layer_bwd.restype = None
        lib.orc_bwd_tokens.argtypes = [i32, i32, i32, i32, i32, p, p, p, p, p, p, p, i64, p, p]
        lib.orc_bwd_tokens.restype = None
        lib.orc_wgrad_elems.argtypes = [i64, i32, i32, i32, i32, i32, i32] + [p] * 6 + [p, i64, p, p, i64, p, p, p]
        lib.orc_e4m3_value.argtypes = [i32]
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
        lib.orc_e4m3_encode.restype = i32
        lib.orc_mx_quantize.argtypes = [p, i64, i32, p, p]
        lib.orc_mx_quantize_f64.argtypes = [p, i64, i32, p, p]
        lib.orc_mx_expert_ffn_rows.argtypes = [i32, i32, i32] + [p] * 7 + [p, i64, p, p, p, p, p, p]
        lib.orc_mx_layer_fwd_tokens.argtypes = [i32, i32, i32, i32, i32] + [p] * 8 + [p, i64, p]
        lib.orc_wgrad_elems.restype = None
        lib.orc_mx_bwd_tokens.argtypes = [i32, i32, i32, i32, i32] + [p] * 11 + [p, i64, p, p, p]
        lib.orc_mx_bwd_tokens.restype = None
        lib.orc_mx_wgrad_elems.argtypes = [i32, i32, i32, i32, i32, i32] + [p] * 12 + [p, i64, p, p, i64, p, p, p]
        lib.orc_mx_wgrad_elems.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 operands are passed as their uint16 bit patterns")
    return np.ascontiguousarray(a)


def capacity_rows(P: int, Np: int, K: int, L: int, pad: int = 256) -> int:
    """Worst-case dispatched rows: P*Np*K + L*(pad-1)."""
    return int(_load().orc_capacity_rows(P, Np, K, L, pad))


def minibatch_floor(C: int, bm: int, bn: int, H: int, I: int) -> int:
    """T >= 2*C*bm*bn / min(2I, H), rounded up (Mixture-of-Kittens notes, section 3)."""
    return int(_load().orc_minibatch_floor(C, bm, bn, H, I))


class Schedule:
    """Result of a schedule: counts [L][P], seg_off [L+1], phi [npad][2],
    route_row [P][Np][K], npad, and instrumentation stats."""

    def __init__(self, counts, seg_off, phi, route_row, npad, stats):
        self.counts = counts
        self.seg_off = seg_off
        self.phi = phi
        self.route_row = route_row
        self.npad = npad
        self.stats = stats


def _schedule_call(fn_name: str, routes: np.ndarray, L: int, base: int, pad: int, NT: int | None):
    routes = _i32(routes)
    P, Np, K = routes.shape
    cap = capacity_rows(P, Np, K, L, pad)
    counts = np.zeros((L, P), np.int32)
    seg_off = np.zeros(L + 1, np.int32)
    phi = np.zeros((max(cap, 1), 2), np.int32)
    route_row = np.zeros((P, Np, K), np.int32)
    lib = _load()
    if fn_name == "counting":
        stats = np.zeros(2, np.int64)
        npad = lib.orc_schedule_counting(P, Np, K, L, base, pad, NT, _ptr(routes), _ptr(counts),
                                         _ptr(seg_off), _ptr(phi), cap, _ptr(route_row), _ptr(stats))
        st = {"route_reads": int(stats[0]), "counters": int(stats[1])}
    else:
        reads = np.zeros(1, np.int64)
        fn = lib.orc_schedule if fn_name == "plain" else lib.orc_schedule_rescan
        npad = fn(P, Np, K, L, base, pad, _ptr(routes), _ptr(counts), _ptr(seg_off), _ptr(phi), cap,
                  _ptr(route_row), _ptr(reads))
        st = {"route_reads": int(reads[0])}
    if npad < 0:
        raise RuntimeError("oracle schedule: capacity exceeded")
    return Schedule(counts, seg_off, phi[:npad].copy(), route_row, int(npad), st)


def schedule(routes: np.ndarray, L: int, base: int = 0, pad: int = 256) -> Schedule:
    """Plain definition of the pull schedule (position formula, two passes)."""
    return _schedule_call("plain", routes, L, base, pad, None)


def schedule_counting(routes: np.ndarray, L: int, base: int = 0, pad: int = 256, NT: int = 1024) -> Schedule:
    """The four counting-sort stages with NT logical threads per partition."""
    return _schedule_call("counting", routes, L, base, pad, NT)


def schedule_rescan(routes: np.ndarray, L: int, base: int = 0, pad: int = 256) -> Schedule:
    """The older per-(expert, peer) rescanning scheduler: lists merged round-robin."""
    return _schedule_call("rescan", routes, L, base, pad, None)


def invalid_ids(routes: np.ndarray, E: int) -> int:
    """Number of route ids outside [0, E) (never local; counted on the device)."""
    routes = _i32(routes)
    return int(_load().orc_invalid_ids(routes.size, E, _ptr(routes)))


def dispatch(X: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Xd[row] = X[phi.part][phi.tok] (bf16 bits), zero rows for padding."""
    X = _u16(X)
    P, Np, H = X.shape
    phi = _i32(phi)
    npad = phi.shape[0]
    Xd = np.zeros((npad, H), np.uint16)
    _load().orc_dispatch(Np, H, _ptr(X), _ptr(phi), npad, _ptr(Xd))
    return Xd


def expert_ffn_rows(seg_off, Xd, W13, W2, rows=None, want=("HU", "A", "Y")):
    """SwiGLU expert FFN of the listed dispatched rows (default: all rows).

    Returns a dict with the requested double arrays HU [n][2I], A [n][I], Y [n][H]."""
    Xd, W13, W2 = _u16(Xd), _u16(W13), _u16(W2)
    seg_off = _i32(seg_off)
    L, twoI, H = W13.shape
    I = twoI // 2
    rows = np.arange(Xd.shape[0], dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    n = rows.shape[0]
    HU = np.zeros((n, 2 * I)) if "HU" in want else None
    A = np.zeros((n, I)) if "A" in want else None
    Y = np.zeros((n, H)) if "Y" in want else None
    _load().orc_expert_ffn_rows(L, H, I, _ptr(seg_off), _ptr(Xd), _ptr(W13), _ptr(W2), _ptr(rows), n,
                                _ptr(HU), _ptr(A), _ptr(Y))
    return {"HU": HU, "A": A, "Y": Y}


def combine(route_row, w, Y_rows, yrow_index=None, tokens=None):
    """out[g] = sum_j w[g][j] * Y[route_row[g][j]] over local slots, ascending j."""
    route_row = _i32(route_row)
    P, Np, K = route_row.shape
    w = np.ascontiguousarray(w, np.float32)
    Y_rows = np.ascontiguousarray(Y_rows, np.float64)
    H = Y_rows.shape[1]
    if yrow_index is None:
        yrow_index = np.arange(Y_rows.shape[0], dtype=np.int64)
    yrow_index = np.ascontiguousarray(yrow_index, np.int64)
    tokens = np.arange(P * Np, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
    out = np.zeros((tokens.shape[0], H))
    _load().orc_combine_tokens(Np, K, H, _ptr(route_row), _ptr(w), _ptr(Y_rows), _ptr(yrow_index),
                               _ptr(tokens), tokens.shape[0], _ptr(out))
    return out


def layer_fwd_tokens(routes, w, X, W13, W2, L: int, base: int = 0, tokens=None):
    """Forward output per token straight from the definition (no schedule)."""
    routes = _i32(routes)
    P, Np, K = routes.shape
    w = np.ascontiguousarray(w, np.float32)
    X, W13, W2 = _u16(X), _u16(W13), _u16(W2)
    H = X.shape[-1]
    I = W13.shape[1] // 2
    tokens = np.arange(P * Np, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
    out = np.zeros((tokens.shape[0], H))
    _load().orc_layer_fwd_tokens(K, L, base, H, I, _ptr(routes), _ptr(w), _ptr(X), _ptr(W13), _ptr(W2),
                                 _ptr(tokens), tokens.shape[0], _ptr(out))
    return out


def layer_bwd(routes, w, X, W13, W2, dOut, L: int, base: int = 0):
    """Full backward: dict of dX [P][Np][H], dW13 [L][2I][H], dW2 [L][H][I], dw [P][Np][K]."""
    routes = _i32(routes)
    P, Np, K = routes.shape
    w = np.ascontiguousarray(w, np.float32)
    X, W13, W2, dOut = _u16(X), _u16(W13), _u16(W2), _u16(dOut)
    H = X.shape[-1]
    I = W13.shape[1] // 2
    dX = np.zeros((P, Np, H))
    dW13 = np.zeros((L, 2 * I, H))
    dW2 = np.zeros((L, H, I))
    dw = np.zeros((P, Np, K))
    _load().orc_layer_bwd(P * Np, K, L, base, H, I, _ptr(routes), _ptr(w), _ptr(X), _ptr(W13), _ptr(W2),
                          _ptr(dOut), _ptr(dX), _ptr(dW13), _ptr(dW2), _ptr(dw))
    return {"dX": dX, "dW13": dW13, "dW2": dW2, "dw": dw}


def bwd_tokens(routes, w, X, W13, W2, dOut, L: int, base: int, tokens):
    """dX rows and dw rows of the listed tokens."""
    routes = _i32(routes)
    P, Np, K = routes.shape
    w = np.ascontiguousarray(w, np.float32)
    X, W13, W2, dOut = _u16(X), _u16(W13), _u16(W2), _u16(dOut)
    H = X.shape[-1]
    I = W13.shape[1] // 2
    tokens = np.ascontiguousarray(tokens, np.int64)
    dX = np.zeros((tokens.shape[0], H))
    dw = np.zeros((tokens.shape[0], K))
    _load().orc_bwd_tokens(K, L, base, H, I, _ptr(routes), _ptr(w), _ptr(X), _ptr(W13), _ptr(W2), _ptr(dOut),
                           _ptr(tokens), tokens.shape[0], _ptr(dX), _ptr(dw))
    return dX, dw


def wgrad_elems(routes, w, X, W13, W2, dOut, L: int, base: int, expert: int, w13_elems, w2_elems,
                with_abs: bool = False):
    """Listed elements of dW13[expert] ((n, k) pairs) and dW2[expert] ((m, n)
    pairs); with_abs also returns, per element, the sum of its terms' absolute
    values (the scale of the error that roundings of the terms can cause)."""
    routes = _i32(routes)
    P, Np, K = routes.shape
    w = np.ascontiguousarray(w, np.float32)
    X, W13, W2, dOut = _u16(X), _u16(W13), _u16(W2), _u16(dOut)
    H = X.shape[-1]
    I = W13.shape[1] // 2
    e13 = np.ascontiguousarray(np.asarray(w13_elems, np.int64).reshape(-1, 2))
    e2 = np.ascontiguousarray(np.asarray(w2_elems, np.int64).reshape(-1, 2))
    g13 = np.zeros(e13.shape[0])
    g2 = np.zeros(e2.shape[0])
    a13 = np.zeros(e13.shape[0]) if with_abs else None
    a2 = np.zeros(e2.shape[0]) if with_abs else None
    _load().orc_wgrad_elems(P * Np, K, L, base, H, I, expert, _ptr(routes), _ptr(w), _ptr(X), _ptr(W13), _ptr(W2),
                            _ptr(dOut), _ptr(e13), e13.shape[0], _ptr(g13), _ptr(e2), e2.shape[0], _ptr(g2),
                            _ptr(a13), _ptr(a2))
    return (g13, g2, a13, a2) if with_abs else (g13, g2)


# ---------------------------------------------------------------------------
# MXFP8 (OCP Microscaling: 32-element blocks along the reduction dimension,
# E8M0 scale 2^(floor(log2 amax) - 8), FP8 E4M3 elements rounded to nearest
# even and saturated at +-448).
# ---------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def e4m3_encode(y: float) -> int:
    return _load().orc_e4m3_encode(float(y))


def e4m3_table() -> np.ndarray:
    """Values of the 256 E4M3 codes (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)])


def mx_quantize(x: np.ndarray):
    """Row-wise MX quantization of bf16 bits [..., K] -> (codes uint8 [..., K],
    scale bytes uint8 [..., K/32])."""
    x = _u16(x)
    K = x.shape[-1]
    rows = x.size // K
    q = np.zeros(x.shape, np.uint8)
    s = np.zeros(x.shape[:-1] + (K // 32,), np.uint8)
    _load().orc_mx_quantize(_ptr(x), rows, K, _ptr(q), _ptr(s))
    return q, s


def mx_quantize_f64(x: np.ndarray):
    x = np.ascontiguousarray(x, np.float64)
    K = x.shape[-1]
    q = np.zeros(x.shape, np.uint8)
    s = np.zeros(x.shape[:-1] + (K // 32,), np.uint8)
    _load().orc_mx_quantize_f64(_ptr(x), x.size // K, K, _ptr(q), _ptr(s))
    return q, s


def mx_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Double values of MX codes and scale bytes (blocks of 32 along the last axis)."""
    t = e4m3_table()
    v = t[np.asarray(q, np.int64)]
    sc = np.repeat(np.ldexp(1.0, np.asarray(s, np.int64) - 127), 32, axis=-1)
    return v * sc


def mx_dispatch(Xq: np.ndarray, Xs: np.ndarray, phi: np.ndarray):
    """MX codes and scales of the dispatched rows: row i = X row phi[i]
    (part * Np + tok); padding rows get code 0 and scale byte 0."""
    Xq, Xs = np.asarray(Xq, np.uint8), np.asarray(Xs, np.uint8)
    P, Np, H = Xq.shape
    phi = _i32(phi)
    real = phi[:, 0] >= 0
    src = (phi[:, 0].astype(np.int64) * Np + phi[:, 1]).clip(min=0)
    q = np.where(real[:, None], Xq.reshape(-1, H)[src], 0).astype(np.uint8)
    s = np.where(real[:, None], Xs.reshape(-1, H // 32)[src], 0).astype(np.uint8)
    return q, s


def mx_expert_ffn_rows(seg_off, Xdq, Xds, W13q, W13s, W2q, W2s, rows=None, with_hu=False):
    """MXFP8 expert FFN of the listed dispatched rows: dict with A (double
    [n][I], before quantization), Aq / As (its MX codes and scales) and Y
    (double [n][H], from the quantized A).  with_hu adds HU (double [n][2I]:
    h then u) and HUabs (the sums of the magnitudes of the terms of each h and
    u, which scale any accumulation error in them)."""
    seg_off = _i32(seg_off)
    arrs = [np.ascontiguousarray(a, np.uint8) for a in (Xdq, Xds, W13q, W13s, W2q, W2s)]
    Xdq, Xds, W13q, W13s, W2q, W2s = arrs
    L, twoI, H = W13q.shape
    I = twoI // 2
    rows = np.arange(Xdq.shape[0], dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    n = rows.shape[0]
    A = np.zeros((n, I))
    Aq = np.zeros((n, I), np.uint8)
    As = np.zeros((n, I // 32), np.uint8)
    Y = np.zeros((n, H))
    HU = np.zeros((n, 2 * I)) if with_hu else None
    HUabs = np.zeros((n, 2 * I)) if with_hu else None
    _load().orc_mx_expert_ffn_rows(L, H, I, _ptr(seg_off), *[_ptr(a) for a in arrs], _ptr(rows), n, _ptr(A),
                                   _ptr(Aq), _ptr(As), _ptr(Y), _ptr(HU), _ptr(HUabs))
    r = {"A": A, "Aq": Aq, "As": As, "Y": Y}
    if with_hu:
        r["HU"], r["HUabs"] = HU, HUabs
    return r


def mx_layer_fwd_tokens(routes, w, Xq, Xs, W13q, W13s, W2q, W2s, L: int, base: int = 0, tokens=None):
    """MXFP8 forward output per token straight from the definition."""
    routes = _i32(routes)
    P, Np, K = routes.shape
    w = np.ascontiguousarray(w, np.float32)
    arrs = [np.ascontiguousarray(a, np.uint8) for a in (Xq, Xs, W13q, W13s, W2q, W2s)]
    H = arrs[0].shape[-1]
    I = arrs[2].shape[1] // 2
    tokens = np.arange(P * Np, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
    out = np.zeros((tokens.shape[0], H))
    _load().orc_mx_layer_fwd_tokens(K, L, base, H, I, _ptr(routes), _ptr(w), *[_ptr(a) for a in arrs],
                                    _ptr(tokens), tokens.shape[0], _ptr(out))
    return out


def mx_transpose_quantize(W: np.ndarray):
    """MX quantization of bf16 bits [..., R, C] along R: codes [..., C, R] and
    scale bytes [..., C, R/32] (each column of W quantized in blocks of 32
    consecutive rows)."""
    return mx_quantize(np.ascontiguousarray(np.swapaxes(_u16(W), -1, -2)))


def mx_weights_t(W13: np.ndarray, W2: np.ndarray):
    """The backward's MX weights: W2 columns along H ([L][I][H]) for the down
    dgrad, W13 columns along 2I ([L][H][2I]) for the gate/up dgrad."""
    W2tq, W2ts = mx_transpose_quantize(W2)
    W13tq, W13ts = mx_transpose_quantize(W13)
    return {"W2tq": W2tq, "W2ts": W2ts, "W13tq": W13tq, "W13ts": W13ts}


def mx_bwd_tokens(routes, w, Xq, Xs, W13q, W13s, wt, dOut, L: int, base: int = 0, tokens=None,
                  with_abs: bool = False):
    """MXFP8 backward, token side: dX rows (double [n][H]) and dw rows ([n][K])
    of the listed tokens.  Xq/Xs, W13q/W13s are the forward's MX operands; wt
    is mx_weights_t(W13, W2).  with_abs also returns the sums |dA'[i] a[i]|."""
    routes = _i32(routes)
    P, Np, K = routes.shape
    w = np.ascontiguousarray(w, np.float32)
    Xq, Xs, W13q, W13s = (np.ascontiguousarray(a, np.uint8) for a in (Xq, Xs, W13q, W13s))
    t = [np.ascontiguousarray(wt[k], np.uint8) for k in ("W2tq", "W2ts", "W13tq", "W13ts")]
    dOut = _u16(dOut)
    H = Xq.shape[-1]
    I = W13q.shape[1] // 2
    tokens = np.arange(P * Np, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
    n = tokens.shape[0]
    dX = np.zeros((n, H))
    dw = np.zeros((n, K))
    dwabs = np.zeros((n, K)) if with_abs else None
    _load().orc_mx_bwd_tokens(K, L, base, H, I, _ptr(routes), _ptr(w), _ptr(Xq), _ptr(Xs), _ptr(W13q), _ptr(W13s),
                              *[_ptr(a) for a in t], _ptr(dOut), _ptr(tokens), n, _ptr(dX), _ptr(dw), _ptr(dwabs))
    return (dX, dw, dwabs) if with_abs else (dX, dw)


def mx_wgrad_elems(sched, routes, w, X, Xq, Xs, W13q, W13s, wt, dOut, expert: int, w13_elems, w2_elems,
                   with_abs: bool = False):
    """Listed elements of the MX backward's dW13[expert] ((nn, k) pairs) and
    dW2[expert] ((m, i) pairs); sched is oracle.schedule(routes, ...) of the
    same routing (its table fixes the row blocks).  with_abs also returns the
    sums of the terms' magnitudes."""
    routes = _i32(routes)
    P, Np, K = routes.shape
    w = np.ascontiguousarray(w, np.float32)
    X, dOut = _u16(X), _u16(dOut)
    Xq, Xs, W13q, W13s = (np.ascontiguousarray(a, np.uint8) for a in (Xq, Xs, W13q, W13s))
    W2tq, W2ts = (np.ascontiguousarray(wt[k], np.uint8) for k in ("W2tq", "W2ts"))
    L, twoI, H = W13q.shape
    I = twoI // 2
    e13 = np.ascontiguousarray(np.asarray(w13_elems, np.int64).reshape(-1, 2))
    e2 = np.ascontiguousarray(np.asarray(w2_elems, np.int64).reshape(-1, 2))
    g13, g2 = np.zeros(e13.shape[0]), np.zeros(e2.shape[0])
    a13 = np.zeros(e13.shape[0]) if with_abs else None
    a2 = np.zeros(e2.shape[0]) if with_abs else None
    _load().orc_mx_wgrad_elems(Np, K, L, H, I, expert, _ptr(_i32(sched.seg_off)), _ptr(_i32(sched.phi)),
                               _ptr(_i32(sched.route_row)), _ptr(w), _ptr(X), _ptr(Xq), _ptr(Xs), _ptr(W13q),
                               _ptr(W13s), _ptr(W2tq), _ptr(W2ts), _ptr(dOut), _ptr(e13), e13.shape[0], _ptr(g13),
                               _ptr(e2), e2.shape[0], _ptr(g2), _ptr(a13), _ptr(a2))
    return (g13, g2, a13, a2) if with_abs else (g13, g2)


def _bf16_via_f32(x):
    """Round doubles to float, then to bf16 with ties to even (the rounding
    the kernels apply to the values they keep in bf16)."""
    f = np.asarray(x, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


def _bf16_values(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _colq(M):
    """MX codes and scales of the columns of M [rows][C] along the rows
    (codes [C][rows], scales [C][rows/32])."""
    return mx_quantize_f64(np.ascontiguousarray(np.asarray(M, np.float64).T))


def mx_layer_bwd(routes, w, X, W13, W2, dOut, L: int, base: int = 0, experts=None):
    """The MXFP8 backward in matrix form (the reading of moe_oracle.c's MXFP8
    backward section): per local expert segment of oracle.schedule's table,
    the forward (h, u from the MX codes of X and W13; a = silu(h) u, its row
    codes), then dA' = dO . W2 (dO rows along H, W2 columns along H),
    dw = dA' . a, dHU = bf16(w dA' u silu'(h), w dA' silu(h)) with h, u as
    bf16, dXd = dHU . W13 (dHU rows along 2I, W13 columns along 2I), and the
    weight gradients from column codes along the segment's rows:
    dW2 = (bf16(w dO))^T a, dW13 = dHU^T Xd.  experts (default all) limits
    the segments computed; the token side (dX, dw) sums only their rows.
    Returns dict: 'sched', 'dX' [P*Np][H], 'dw' [P*Np][K], and per computed
    expert l a dict 'seg'[l] with rows, HU (double, exact), a (dequantized
    codes; a_exact before quantization; HUabs the sums of the magnitudes of
    h's and u's terms), dAp, dHU (bf16 values), dHUq/dHUs (row codes), dXd, the column
    codes dHUT, aT, XdT, dOwT (each (codes [C][rows], scales)) and dW13, dW2.
    Dense numpy products in double; for shapes whose segments fit in memory."""
    routes = _i32(routes)
    P, Np, K = routes.shape
    X, W13, W2, dOut = _u16(X), _u16(W13), _u16(W2), _u16(dOut)
    H = X.shape[-1]
    I = W13.shape[1] // 2
    w = np.asarray(w, np.float32).reshape(-1, K)
    s = schedule(routes, L, base)
    rr = s.route_row.reshape(-1, K)
    Xdeq = mx_dequantize(*mx_quantize(X)).reshape(-1, H)
    dOq = mx_dequantize(*mx_quantize(dOut)).reshape(-1, H)
    dOv = _bf16_values(dOut).reshape(-1, H)
    Xv = _bf16_values(X).reshape(-1, H)
    dX = np.zeros((P * Np, H))
    dw = np.zeros((P * Np, K))
    seg = {}
    for l in (range(L) if experts is None else experts):
        r0, r1 = int(s.seg_off[l]), int(s.seg_off[l + 1])
        if r1 == r0:
            continue
        rows = np.arange(r0, r1)
        ph = s.phi[rows]
        re = ph[:, 0] >= 0
        g = np.where(re, ph[:, 0].astype(np.int64) * Np + ph[:, 1], 0)
        slot = np.full(rows.size, -1, np.int64)
        tk, jk = np.nonzero((rr >= r0) & (rr < r1))
        slot[rr[tk, jk] - r0] = jk
        wr = np.where(re, w[g, np.maximum(slot, 0)].astype(np.float64), 0.0)
        W13deq = mx_dequantize(*mx_quantize(W13[l]))                       # [2I][H]
        W2t = mx_dequantize(*mx_transpose_quantize(W2[l]))                 # [I][H]
        W13t = mx_dequantize(*mx_transpose_quantize(W13[l]))               # [H][2I]
        Xg = np.where(re[:, None], Xdeq[g], 0.0)
        HU = Xg @ W13deq.T
        hh, uu = HU[:, :I], HU[:, I:]
        a_exact = hh / (1.0 + np.exp(-hh)) * uu
        Aq, As = mx_quantize_f64(a_exact)
        a = mx_dequantize(Aq, As)
        hb, ub = _bf16_via_f32(hh), _bf16_via_f32(uu)
        dAp = np.where(re[:, None], dOq[g], 0.0) @ W2t.T
        dA = wr[:, None] * dAp
        sg = 1.0 / (1.0 + np.exp(-hb))
        dHU = np.concatenate([_bf16_via_f32(dA * ub * sg * (1.0 + hb * (1.0 - sg))), _bf16_via_f32(dA * hb * sg)], 1)
        dHUq, dHUs = mx_quantize_f64(dHU)
        dXd = mx_dequantize(dHUq, dHUs) @ W13t.T
        dwr = (dAp * a).sum(1)
        for k in np.nonzero(re)[0]:
            dX[g[k]] += dXd[k]
            dw[g[k], slot[k]] = dwr[k]
        dOw = np.where(re[:, None], _bf16_via_f32(wr[:, None] * dOv[g]), 0.0)
        XdT, dOwT, aT, dHUT = (_colq(M) for M in (np.where(re[:, None], Xv[g], 0.0), dOw, a, dHU))
        seg[l] = {"rows": rows, "HU": HU, "HUabs": np.abs(Xg) @ np.abs(W13deq).T, "a_exact": a_exact, "a": a,
                  "Aq": Aq, "As": As, "dAp": dAp, "dHU": dHU, "dHUq": dHUq,
                  "dHUs": dHUs, "dXd": dXd, "XdT": XdT, "dOwT": dOwT, "aT": aT, "dHUT": dHUT, "W13t": W13t,
                  "dW2": mx_dequantize(*dOwT) @ mx_dequantize(*aT).T,
                  "dW13": mx_dequantize(*dHUT) @ mx_dequantize(*XdT).T}
    return {"sched": s, "dX": dX, "dw": dw, "seg": seg}


# ---------------------------------------------------------------------------
# Macrobatch ring ("Beyond Peak TFLOPs" section 2.B; Mixture-of-Kittens notes,
# section 4).  The ring changes where rows live and in which order
# macrobatches run, not what the layer computes: its outputs are those of
# layer_fwd_tokens / layer_bwd.
# ---------------------------------------------------------------------------

def macrobatch_schedules(routes: np.ndarray, L: int, mb_tokens: int, base: int = 0, pad: int = 256):
    """One table per macrobatch: macrobatch m is tokens [m*mb_tokens,
    (m+1)*mb_tokens) of every partition, scheduled on its own (its Phi holds
    the token's index inside the window)."""
    P, Np, K = routes.shape
    assert Np % mb_tokens == 0
    return [schedule(np.ascontiguousarray(routes[:, m * mb_tokens:(m + 1) * mb_tokens]), L, base, pad)
            for m in range(Np // mb_tokens)]


def ring_walk(M: int, S: int, reverse: bool = True):
    """The forward's walk over M macrobatches through S ring slots, as a plain
    simulation: walk step i takes macrobatch M-1-i (reverse) or i and slot
    i % S, evicting the slot's previous occupant.  Returns the walk
    [(m, slot)], the macrobatches still resident afterwards {m: slot}, and the
    ones the backward (token order m = 0, 1, ...) must replay."""
    walk = [((M - 1 - i) if reverse else i, i % S) for i in range(M)]
    resident = {}
    for m, slot in walk:
        resident = {k: v for k, v in resident.items() if v != slot}
        resident[m] = slot
    replay = [m for m in range(M) if m not in resident]
    return walk, resident, replay


# ---------------------------------------------------------------------------
# Shared expert ("Beyond Peak TFLOPs" section 2.C; Mixture-of-Kittens notes,
# section 5): a dense SwiGLU expert applied to every token, its output added to
# the routed combine.
# ---------------------------------------------------------------------------

def shared_ffn_tokens(X, W13s, W2s, tokens=None):
    """S[g] = W2s (silu(W1s x_g) * (W3s x_g)) for the listed tokens (default all),
    as the single-expert FFN over the token rows in their own order."""
    X = _u16(X)
    H = X.shape[-1]
    Xr = np.ascontiguousarray(X.reshape(-1, H))
    seg = np.array([0, Xr.shape[0]], np.int32)
    return expert_ffn_rows(seg, Xr, _u16(W13s)[None], _u16(W2s)[None], rows=tokens, want=("Y",))["Y"]


def layer_fwd_tokens_shared(routes, w, X, W13, W2, W13s, W2s, L: int, base: int = 0, tokens=None):
    """Layer output with a shared expert: routed combine + shared FFN, per token."""
    return (layer_fwd_tokens(routes, w, X, W13, W2, L=L, base=base, tokens=tokens)
            + shared_ffn_tokens(X, W13s, W2s, tokens=tokens))
