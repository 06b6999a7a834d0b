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
    return {"counts": counts.cpu().numpy(), "seg_off": seg_off.cpu().numpy(), "phi": phi.cpu().numpy(),
            "route_row": route_row.cpu().numpy(), "cap": cap}
