"""Seeded synthetic inputs shaped like the workloads on the Mixture-of-Kittens pages.

This module only draws random data (numpy ``PCG64``); it holds none of the
layer's arithmetic, so both the HIP path and the CPU oracle can be fed from it.
bf16 tensors are returned as their uint16 bit patterns (round-to-nearest-even
of a float32 draw).

Routing generators (all return ``routes int32 [P][Np][K]`` and router weights
``w float32 [P][Np][K]``):
  uniform      K distinct ids per token, uniform over distinct sets
  topk_logits  ids = top-K of N(0,1) logits over E experts, w = softmax of the
               selected logits (the small forward configuration)
  zipf(s)      expert popularity proportional to rank^-s over a seeded rank
               permutation, K distinct ids per token by Gumbel-top-K
  balanced     e(g, j) = (sigma(g) + j*E/K) mod E with sigma a seeded permutation
               of the P*Np tokens and the slot order shuffled per token: exactly
               one route per token lands in each E/K-wide block of ids
  hot          nhot local hot experts take hot_slots of each token's K slots
               (each hot expert gets exactly P*Np*hot_slots/nhot routes), the
               other slots Zipf(s) over the remaining experts
"""
from __future__ import annotations

import numpy as np


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    # finite and infinite inputs cannot overflow 32 bits here (max 0xFF807FFF)
    r = ((np.where(nan, np.uint32(0), u) + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def _softmax_sorted_weights(rng: np.random.Generator, n: int, K: int) -> np.ndarray:
    z = -np.sort(-rng.standard_normal(size=(n, K), dtype=np.float32), axis=1)
    z = z - z[:, :1]
    e = np.exp(z.astype(np.float64))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def routes_uniform(rng, P: int, Np: int, E: int, K: int):
    """K distinct uniform ids per token (rejection of rows with repeats)."""
    n = P * Np
    ids = rng.integers(0, E, size=(n, K), dtype=np.int64)
    while True:
        s = np.sort(ids, axis=1)
        bad = np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0] if K > 1 else np.zeros(0, np.int64)
        if bad.size == 0:
            break
        ids[bad] = rng.integers(0, E, size=(bad.size, K), dtype=np.int64)
    w = _softmax_sorted_weights(rng, n, K)
    return ids.astype(np.int32).reshape(P, Np, K), w.reshape(P, Np, K)


def routes_topk_logits(rng, P: int, Np: int, E: int, K: int):
    """ids = top-K of N(0,1) logits (descending), w = softmax over the K selected logits."""
    n = P * Np
    logits = rng.standard_normal(size=(n, E), dtype=np.float32)
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    sel = np.take_along_axis(logits, idx, axis=1).astype(np.float64)
    e = np.exp(sel - sel[:, :1])
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx.astype(np.int32).reshape(P, Np, K), w.reshape(P, Np, K)


def _gumbel_topk(rng, n: int, logp: np.ndarray, K: int, chunk: int = 8192) -> np.ndarray:
    E = logp.shape[0]
    out = np.empty((n, K), np.int64)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        g = rng.gumbel(size=(m, E)).astype(np.float32) + logp[None, :]
        part = np.argpartition(-g, K - 1, axis=1)[:, :K]
        order = np.argsort(-np.take_along_axis(g, part, axis=1), axis=1, kind="stable")
        out[s:s + m] = np.take_along_axis(part, order, axis=1)
    return out


def zipf_logp(rng, E: int, s: float) -> np.ndarray:
    ranks = rng.permutation(E) + 1
    p = ranks.astype(np.float64) ** (-s)
    return np.log(p / p.sum()).astype(np.float32)


def routes_zipf(rng, P: int, Np: int, E: int, K: int, s: float):
    logp = zipf_logp(rng, E, s)
    ids = _gumbel_topk(rng, P * Np, logp, K)
    w = _softmax_sorted_weights(rng, P * Np, K)
    return ids.astype(np.int32).reshape(P, Np, K), w.reshape(P, Np, K)


def routes_balanced(rng, P: int, Np: int, E: int, K: int):
    """e(g, j) = (sigma(g) + j*E/K) mod E, slot order shuffled per token."""
    if E % K:
        raise ValueError("balanced routing needs K | E")
    n = P * Np
    sigma = rng.permutation(n).astype(np.int64)
    ids = (sigma[:, None] + np.arange(K, dtype=np.int64)[None, :] * (E // K)) % E
    perm = np.argsort(rng.random(size=(n, K)), axis=1)
    ids = np.take_along_axis(ids, perm, axis=1)
    w = _softmax_sorted_weights(rng, n, K)
    return ids.astype(np.int32).reshape(P, Np, K), w.reshape(P, Np, K)


def routes_hot(rng, P: int, Np: int, E: int, K: int, L: int, base: int = 0,
               nhot: int = 4, hot_slots: int = 2, s: float = 1.5):
    """Adversarial skew: nhot local experts share hot_slots of every token's K slots
    (tokens alternate between hot pairs by a seeded permutation, so each hot
    expert receives exactly n*hot_slots/nhot routes); the remaining K-hot_slots
    slots are Zipf(s) over the other E-nhot experts.  Slots shuffled per token."""
    n = P * Np
    hot = base + rng.choice(L, size=nhot, replace=False)
    groups = nhot // hot_slots
    sigma = rng.permutation(n)
    grp = sigma % groups
    hot_ids = hot.reshape(groups, hot_slots)[grp]
    others = np.setdiff1d(np.arange(E), hot)
    logp = zipf_logp(rng, others.size, s)
    cold = others[_gumbel_topk(rng, n, logp, K - hot_slots)]
    ids = np.concatenate([hot_ids, cold], axis=1)
    perm = np.argsort(rng.random(size=(n, K)), axis=1)
    ids = np.take_along_axis(ids, perm, axis=1)
    w = _softmax_sorted_weights(rng, n, K)
    return ids.astype(np.int32).reshape(P, Np, K), w.reshape(P, Np, K), np.sort(hot)


def make_routes(kind: str, rng, P: int, Np: int, E: int, K: int, L: int = 0, base: int = 0, s: float = 1.2):
    if kind == "uniform":
        return routes_uniform(rng, P, Np, E, K)
    if kind == "topk":
        return routes_topk_logits(rng, P, Np, E, K)
    if kind == "zipf":
        return routes_zipf(rng, P, Np, E, K, s)
    if kind == "balanced":
        return routes_balanced(rng, P, Np, E, K)
    if kind == "hot":
        r, w, _ = routes_hot(rng, P, Np, E, K, L, base, s=s)
        return r, w
    raise ValueError(kind)


def make_layer_inputs(seed: int, P: int, Np: int, E: int, K: int, L: int, H: int, I: int,
                      routing: str = "uniform", base: int = 0, x_std: float = 0.02,
                      w_std: float = 0.02, s: float = 1.2, with_grad: bool = False):
    """All forward (and optionally backward) inputs of one layer call."""
    rng = rng_for(seed)
    routes, w = make_routes(routing, rng, P, Np, E, K, L, base, s)
    X = normal_bf16(rng, (P, Np, H), x_std)
    W13 = normal_bf16(rng, (L, 2 * I, H), w_std)
    W2 = normal_bf16(rng, (L, H, I), w_std)
    d = {"routes": routes, "w": w, "X": X, "W13": W13, "W2": W2}
    if with_grad:
        d["dOut"] = normal_bf16(rng, (P, Np, H), x_std)
    return d


def normal_bf16_device(shape, std: float, seed: int, device):
    """Seeded N(0, std^2) bf16 tensor drawn on the GPU (torch's Philox generator).

    For the multi-GB weight tensors of the full-size configurations; the
    oracle receives the same values by copying them back to the host."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(torch.bfloat16)


def make_layer_inputs_device(seed: int, P: int, Np: int, E: int, K: int, L: int, H: int, I: int, device,
                             routing: str = "balanced", base: int = 0, x_std: float = 1.0, w_std: float = 0.02,
                             s: float = 1.2, with_grad: bool = False):
    """Routes and router weights on the host (numpy PCG64), dense tensors drawn
    on the device; returns host routes/w and device X, W13, W2 (and dOut)."""
    rng = rng_for(seed)
    routes, w = make_routes(routing, rng, P, Np, E, K, L, base, s)
    d = {"routes": routes, "w": w,
         "X": normal_bf16_device((P, Np, H), x_std, seed * 8 + 1, device),
         "W13": normal_bf16_device((L, 2 * I, H), w_std, seed * 8 + 2, device),
         "W2": normal_bf16_device((L, H, I), w_std, seed * 8 + 3, device)}
    if with_grad:
        d["dOut"] = normal_bf16_device((P, Np, H), x_std, seed * 8 + 4, device)
    return d


# The five workloads (shapes from the pages: the Kimi-shaped share is
# H=7168, I=2048, 384 experts, top-8, 8 partitions of 7,168 tokens).
CONFIGS = {
    "tiny": dict(P=2, Np=256, E=8, K=2, L=4, H=256, I=128, routing="topk", x_std=0.02),
    "schedule": dict(P=8, Np=7168, E=384, K=8, L=48),
    "mid": dict(P=8, Np=4096, E=64, K=6, L=8, H=2048, I=1024, routing="uniform", x_std=1.0),
    "kimi": dict(P=8, Np=7168, E=384, K=8, L=48, H=7168, I=2048, routing="balanced", x_std=1.0),
    "kimi_bwd": dict(P=8, Np=7168, E=384, K=8, L=48, H=7168, I=2048, routing="hot", x_std=1.0, s=1.5),
}
