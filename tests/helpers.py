"""Shared helpers of the GPU tests: upload/download and error metrics."""
import hashlib

import numpy as np
import torch

from routing_schedule_expert_amd import ops


def dev():
    return torch.device("cuda:0")


def up_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def up(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def rows_rel_l2(got, ref) -> np.ndarray:
    """Per-row rel-L2 (rows = first axis).  A row whose reference is all zero
    scores 0 if the result row is all zero too, else infinity."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    got = got.reshape(got.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    safe = np.where(den > 0, den, 1.0)
    return np.where(den > 0, num / safe, np.where(num > 0, np.inf, 0.0))


def assert_rows(name, got, ref, tol, ids=None):
    """Every row within rel-L2 tol of its reference row; prints the worst row
    (its index in `ids` when given) and the aggregate rel-L2."""
    rel = rows_rel_l2(got, ref)
    if rel.size == 0:
        return
    i = int(np.argmax(rel))
    where = int(ids[i]) if ids is not None else i
    print(f"    {name}: {rel.size} rows, worst row {where} rel-L2 {rel[i]:.2e}, "
          f"aggregate {rel_l2(got, ref):.2e}", flush=True)
    assert rel[i] <= tol, f"{name}: row {where} rel-L2 {rel[i]:.3e} > {tol}"


def assert_elems(name, got, ref, tol):
    """Scalars (dot products that may cancel): |got - ref| <= tol * max(|ref|,
    rms(ref)) for every element; prints the worst one."""
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    if ref.size == 0:
        return
    floor = np.sqrt(np.mean(ref * ref))
    scale = np.maximum(np.abs(ref), floor if floor > 0 else 1.0)
    err = np.abs(got - ref) / scale
    i = int(np.argmax(err))
    print(f"    {name}: {ref.size} elements, worst {i} scaled error {err[i]:.2e}", flush=True)
    assert err[i] <= tol, f"{name}: element {i} got {got[i]!r} want {ref[i]!r} (scaled error {err[i]:.3e})"


def digest(*tensors) -> str:
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


def gpu_schedule(routes: np.ndarray, L: int, base: int = 0, pad: int = 256, E: int | None = None, NT: int = 1024):
    """Run moe_schedule on routes [nb][P][Np][K] (or [P][Np][K]); numpy results."""
    r = routes if routes.ndim == 4 else routes[None]
    nb, P, Np, K = r.shape
    if E is None:
        E = max(int(r.max()) + 1, base + L)
    d = ops.make_desc(P, Np, K, E, L, expert_base=base, pad_rows=pad, sched_threads=NT, num_batches=nb)
    cap = ops.capacity_rows(d)
    rt = up(r.astype(np.int32))
    counts = torch.full((nb, L, P), -7, dtype=torch.int32, device=dev())
    seg_off = torch.full((nb, L + 1), -7, dtype=torch.int32, device=dev())
    phi = torch.full((nb, cap, 2), -7, dtype=torch.int32, device=dev())
    route_row = torch.full((nb, P, Np, K), -7, dtype=torch.int32, device=dev())
    ws = torch.full((ops.workspace_bytes(d, ops.MOE_OP_SCHEDULE),), 0x5A, dtype=torch.uint8, device=dev())
    ops.moe_schedule(d, rt, counts, seg_off, phi, route_row, ws)
    torch.cuda.synchronize()
    inv = ops.read_ws_words(ws, ops.workspace_field(d, ops.MOE_OP_SCHEDULE, ops.MOE_WS_INVALID_IDS), nb)
    return {"counts": counts.cpu().numpy(), "seg_off": seg_off.cpu().numpy(), "phi": phi.cpu().numpy(),
            "route_row": route_row.cpu().numpy(), "cap": cap, "invalid": inv, "E": E}


def local_counts(routes: np.ndarray, L: int, base: int) -> np.ndarray:
    """Local routes of every token (routes [..., K], flattened over tokens)."""
    r = np.asarray(routes).reshape(-1, np.asarray(routes).shape[-1]).astype(np.int64)
    return ((r >= base) & (r < base + L)).sum(axis=1)


def row_tokens(phi: np.ndarray, Np: int) -> np.ndarray:
    """Token index p * Np + t of every table row (-1 on padding rows)."""
    phi = np.asarray(phi).reshape(-1, 2).astype(np.int64)
    return np.where(phi[:, 0] >= 0, phi[:, 0] * Np + phi[:, 1], -1)


def fused_y_rows(routes: np.ndarray, L: int, base: int, phi: np.ndarray) -> np.ndarray:
    """Mask over the table rows of phi: the rows of the routed Y that the fused
    forward (separate launches without chunks, and the MX forward) writes.
    Those are the padding rows and the rows of tokens with two or more local
    routes; a token with one local route gets its output straight from the
    down GEMM's epilogue, and its Y row is not written."""
    Np = np.asarray(routes).shape[-2]
    g = row_tokens(phi, Np)
    n = local_counts(routes, L, base)
    return (g < 0) | (n[np.maximum(g, 0)] >= 2)


def on_dev_mask(mask: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(mask)).to(dev())


def single_route_terms(routes: np.ndarray, w: np.ndarray, L: int, base: int, phi: np.ndarray, rows: np.ndarray):
    """For table rows `rows`: whether the row's token has exactly one local
    route (then the fused forward writes w * Y[row] straight to out[token]),
    the token index, and the router weight of that route."""
    routes = np.asarray(routes)
    K, Np = routes.shape[-1], routes.shape[-2]
    g = row_tokens(phi, Np)[rows]
    r = routes.reshape(-1, K).astype(np.int64)
    local = (r >= base) & (r < base + L)
    gg = np.maximum(g, 0)
    single = (g >= 0) & (local[gg].sum(axis=1) == 1)
    j = np.argmax(local[gg], axis=1)
    wt = np.asarray(w).reshape(-1, K)[gg, j].astype(np.float64)
    return single, g, wt


def expected_single_route_table(routes: np.ndarray, w: np.ndarray, L: int, base: int, phi: np.ndarray) -> np.ndarray:
    """The forward's per-row table of single-route tokens, as int32 pairs
    [npad][2]: (token, bits of its fp32 weight) for a row whose token has
    exactly one local route, (-1, 0) for every other row and padding."""
    rows = np.arange(np.asarray(phi).shape[0])
    single, g, wt = single_route_terms(routes, w, L, base, phi, rows)
    tab = np.zeros((rows.size, 2), np.int32)
    tab[:, 0] = -1
    tab[single, 0] = g[single]
    tab[single, 1] = wt[single].astype(np.float32).view(np.int32)
    return tab
