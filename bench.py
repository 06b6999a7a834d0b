#!/usr/bin/env python3
"""Benchmark of one MI355X's share of the Kimi-shaped MoE layer forward.

One step = one pass of the whole forward hot path through the C ABI
(moe_layer_fwd: counting-sort schedule, pull gather (by default fused into the
gate/up GEMM's operand loads), SwiGLU grouped GEMMs, fixed-order combine) on 8 partitions x 7,168 tokens, 384 experts (48 local),
top-8, H=7168, I=2048, balanced routing (one local route per token), bf16,
inputs resident in HBM.  Prints ONE JSON line:

  value      layer-forward TFLOP/s, algorithmic (6*H*I flop per local route)
  roofline   the dominant kernel (gate/up grouped GEMM + SwiGLU) against the
             bf16 dense MFMA peak; its duration comes from HIP events recorded
             on its own stream around every launch in the timed region
  schedule   the schedule alone on 64 independent routing tensors per call
             (routes/s and compulsory HBM bytes against 8 TB/s)
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload

python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "MoE layer fwd TFLOP/s + MFMA util; schedule routes/s (Kimi shape, 1 GPU)"

KIMI = dict(P=8, Np=7168, E=384, K=8, L=48, H=7168, I=2048)
KERNEL_SOURCES = ("routing_schedule_expert_amd/csrc/gemm.hpp", "routing_schedule_expert_amd/csrc/layer.hpp",
                  "routing_schedule_expert_amd/csrc/common.hpp", "routing_schedule_expert_amd/csrc/wide.hpp")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def profile_fields(name: str):
    """`key: value` lines of a committed rocprofv3 summary under profiles/, or
    None when it is missing or the kernel sources changed since the counters
    were taken (its kernel_source_digest no longer matches)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith((" ", "#", "|", "`")):
            k, v = ln.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return rec


def measured_traffic(kernel: str):
    """HBM bytes per launch (fetched + written) from the committed counter
    summary, or None when it is stale."""
    rec = profile_fields(f"{kernel}_kimi_traffic.md")
    try:
        return int(rec["hbm_bytes_per_launch"]) if rec else None
    except (KeyError, ValueError):
        return None


def measured_mfma_counters():
    """MFMA busy fraction and engine clock of the grouped GEMMs from the
    committed counter summary (SQ_VALU_MFMA_BUSY_CYCLES over active cycles x
    SIMDs, GRBM_GUI_ACTIVE per XCD over the dispatch time), or None when it is
    stale.  Counters cannot be read inside the timed run itself."""
    rec = profile_fields("ffn_gemm_kimi_mfma_util.md")
    if not rec:
        return None
    out = {"source": "profiles/ffn_gemm_kimi_mfma_util.md"}
    for k in ("gateup_mfma_busy", "gateup_clock_ghz", "down_mfma_busy", "down_clock_ghz"):
        try:
            out[k] = float(rec[k])
        except (KeyError, ValueError):
            return None
    return out


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(torch, dev, mib: int):
    """One plain elementwise kernel of known traffic (reads and writes `mib`
    MiB of float32), for scaling the HBM byte counters of a profiled run."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def bench_layer(args, torch, ops, inputs, dev):
    c = KIMI
    h = inputs.make_layer_inputs_device(5, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], dev,
                                        routing="balanced", x_std=1.0)
    d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], c["L"], H=c["H"], I=c["I"])
    routes = torch.from_numpy(h["routes"]).to(dev)
    w = torch.from_numpy(h["w"]).to(dev)
    X, W13, W2 = h["X"], h["W13"], h["W2"]
    bufs = ops.alloc_fwd(d, dev, save_hu=True, save_xd=args.materialize_xd)
    local_routes = int(((h["routes"] >= 0) & (h["routes"] < c["L"])).sum())
    flops = 6.0 * c["H"] * c["I"] * local_routes
    flops_gateup = 4.0 * c["H"] * c["I"] * local_routes
    flops_down = 2.0 * c["H"] * c["I"] * local_routes
    flags = ops.MOE_PERSISTENT if args.persistent else 0

    def step():
        ops.layer_fwd(d, routes, w, X, W13, W2, bufs, flags=flags, chunk_rows=args.chunk_rows)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ops.moe_trace_enable(args.steps * 16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    recs = ops.moe_trace_read(args.steps * 16)
    ops.moe_trace_enable(0)
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    stage_ms = {k: float(np.mean(v)) for k, v in per.items()}
    npad = int(bufs.seg_off[-1].item())
    return dict(d=d, h=h, bufs=bufs, ms_step=ms_step, stage_ms=stage_ms, flops=flops, flops_gateup=flops_gateup,
                flops_down=flops_down, local_routes=local_routes, npad=npad, routes=routes, w=w)


def bench_schedule(args, torch, ops, inputs, dev, nb, kind="uniform", P=8, Np=7168, E=384, K=8, L=48, distinct=8):
    """The schedule alone on `nb` routing tensors per call.  For nb > distinct
    the host draws `distinct` tables and repeats them (the tables are
    independent on the device, so the work is the same)."""
    rng = inputs.rng_for(2 if kind == "uniform" else 3)
    nd = min(nb, distinct)
    if kind == "uniform":
        base = [inputs.routes_uniform(rng, P, Np, E, K)[0] for _ in range(nd)]
    else:
        base = [inputs.routes_zipf(rng, P, Np, E, K, 1.2)[0] for _ in range(nd)]
    r = np.stack([base[i % nd] for i in range(nb)])
    d = ops.make_desc(P, Np, K, E, L, num_batches=nb)
    cap = ops.capacity_rows(d)
    rt = torch.from_numpy(r).to(dev)
    counts = torch.empty((nb, L, P), dtype=torch.int32, device=dev)
    seg_off = torch.empty((nb, L + 1), dtype=torch.int32, device=dev)
    phi = torch.empty((nb, cap, 2), dtype=torch.int32, device=dev)
    route_row = torch.empty_like(rt)
    ws = torch.empty(ops.workspace_bytes(d, ops.MOE_OP_SCHEDULE), dtype=torch.uint8, device=dev)
    for _ in range(3):
        ops.moe_schedule(d, rt, counts, seg_off, phi, route_row, ws)
    reps = max(10, args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        ops.moe_schedule(d, rt, counts, seg_off, phi, route_row, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # per-kernel split from events around each launch (a separate, traced pass)
    ops.moe_trace_enable(reps * 4)
    for _ in range(reps):
        ops.moe_schedule(d, rt, counts, seg_off, phi, route_row, ws)
    torch.cuda.synchronize()
    split = {}
    for name, t in ops.moe_trace_read(reps * 4):
        split.setdefault(name, []).append(t)
    ops.moe_trace_enable(0)
    split = {k: float(np.mean(v)) for k, v in split.items()}
    routes = nb * P * Np * K
    npad = seg_off[:, -1].to(torch.int64).sum().item()
    compulsory = routes * 4 + routes * 4 + npad * 8  # read ids, write route_row, write the table
    two_pass = routes * 4 * 2 + routes * 4 + npad * 8  # as described: the ids are read twice
    local = int(((r >= 0) & (r < L)).sum())
    return dict(nb=nb, routing=kind, P=P, Np=Np, E=E, K=K, L=L, ms=ms, split_ms=split,
                routes_per_s=routes / (ms / 1e3), local_routes=local, dispatched_rows=npad,
                compulsory_bytes=compulsory, gbs=compulsory / (ms / 1e3) / 1e9,
                hbm_frac=compulsory / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                two_pass_bytes=two_pass, two_pass_frac=two_pass / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, routes=r)


def copy_bandwidth(torch, dev, mib: int = 2048, reps: int = 10) -> float:
    """Measured device-to-device streaming rate (GB/s, read + write bytes) of
    one plain elementwise kernel over `mib` MiB, for context beside 8 TB/s."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2.0 * n * 4 / (ms / 1e3) / 1e9


def bench_schedule_sweep(args, torch, ops, inputs, dev):
    """The schedule-only table: Kimi shape (8 partitions x 7,168 tokens, 384
    experts with 48 local, top-8, rows padded to 256) at 1 and 64 routing
    tensors per call, uniform and Zipf s=1.2 routing; then 512 tokens per
    partition, and E in {64, 128, 256, 384} with P = 8 (L = E/8)."""
    copy_gbs = copy_bandwidth(torch, dev)
    rows = []
    cases = [dict(nb=nb, kind=k) for k in ("uniform", "zipf") for nb in (1, 64)]
    cases += [dict(nb=nb, kind="uniform", Np=512) for nb in (1, 64)]
    cases += [dict(nb=nb, kind="uniform", E=e, L=e // 8) for e in (64, 128, 256) for nb in (1, 64)]
    for c in cases:
        print(f"[bench] schedule {c}", file=sys.stderr, flush=True)
        res = bench_schedule(args, torch, ops, inputs, dev, **c)
        res.pop("routes")
        res["frac_of_copy"] = res["gbs"] / copy_gbs
        rows.append(res)
    return {"metric": "schedule routes/s and HBM fraction (compulsory bytes), 1 GPU", "unit": "routes/s",
            "peak_GBs": PEAK_HBM_GBS, "copy_GBs": copy_gbs, "data": "synthetic", "sweep": rows}


def bench_fwd_bwd(args, torch, ops, inputs, dev):
    """Kimi-shaped forward + backward: adversarial routing (Zipf s=1.5 + 4 hot
    local experts taking a quarter of the routes) or balanced routing."""
    c = KIMI
    routing = args.bwd_routing
    h = inputs.make_layer_inputs_device(6, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], dev,
                                        routing=routing, x_std=1.0, s=1.5, with_grad=True)
    d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], c["L"], H=c["H"], I=c["I"])
    routes = torch.from_numpy(h["routes"]).to(dev)
    w = torch.from_numpy(h["w"]).to(dev)
    b = ops.alloc_fwd(d, dev, save_hu=True)
    L, H, I = c["L"], c["H"], c["I"]
    dX = torch.empty_like(h["X"])
    dW13 = torch.empty((L, 2 * I, H), dtype=torch.float32, device=dev)
    dW2 = torch.empty((L, H, I), dtype=torch.float32, device=dev)
    dw = torch.empty((c["P"], c["Np"], c["K"]), dtype=torch.float32, device=dev)
    ws = torch.empty(ops.workspace_bytes(d, ops.MOE_OP_LAYER_BWD), dtype=torch.uint8, device=dev)
    local = int(((h["routes"] >= 0) & (h["routes"] < L)).sum())

    def step():
        ops.layer_fwd(d, routes, w, h["X"], h["W13"], h["W2"], b)
        ops.moe_layer_bwd(d, h["dOut"], routes, w, b.phi, b.route_row, b.seg_off, b.Xd, b.HU, b.A, h["W13"],
                          h["W2"], dX, dW13, dW2, dw, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ops.moe_trace_enable(args.steps * 32)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per = {}
    for name, t in ops.moe_trace_read(args.steps * 32):
        per.setdefault(name, []).append(t)
    ops.moe_trace_enable(0)
    st = {k: float(np.mean(v)) for k, v in per.items()}
    hi = c["H"] * c["I"]
    fl = 18.0 * hi * local
    npad = int(b.seg_off[-1].item())
    return {"metric": f"MoE layer fwd+bwd TFLOP/s (Kimi shape, {'adversarial' if routing == 'hot' else routing} routing, 1 GPU)",
            "value": fl / (ms / 1e3) / 1e12, "unit": "TFLOP/s", "ms_per_step": ms, "steps": args.steps,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "kimi_local_share_fwd_bwd",
                       "routing": "zipf1.5+4hot" if routing == "hot" else routing, "local_routes": local,
                       "dispatched_rows": npad},
            "stage_ms": st,
            "kernel_tflops": {k: v for k, v in {
                "ffn_gateup": 4.0 * hi * local / (st.get("ffn_gateup", 1e9) / 1e3) / 1e12,
                "ffn_down": 2.0 * hi * local / (st.get("ffn_down", 1e9) / 1e3) / 1e12,
                "bwd_down": 2.0 * hi * local / (st.get("bwd_down", 1e9) / 1e3) / 1e12,
                "bwd_gateup": 4.0 * hi * local / (st.get("bwd_gateup", 1e9) / 1e3) / 1e12,
                "bwd_wgrad_rdispatch": 6.0 * hi * local / (st.get("bwd_wgrad_rdispatch", 1e9) / 1e3) / 1e12}.items()}}


def bench_ring(args, torch, ops, inputs, dev):
    """Kimi-shaped share (balanced routing) through the macrobatch ring
    (moe_layer_fwd_ring / moe_layer_bwd_ring) for several (tokens per
    partition per macrobatch, ring slots) settings, beside the ring-less path
    on the same inputs: forward and forward + backward time, dispatched rows
    (each macrobatch pads its own segments), replayed macrobatches and the
    bytes of the row buffers each path keeps."""
    c = KIMI
    h = inputs.make_layer_inputs_device(7, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], dev,
                                        routing="balanced", x_std=1.0, with_grad=True)
    d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], c["L"], H=c["H"], I=c["I"])
    routes = torch.from_numpy(h["routes"]).to(dev)
    w = torch.from_numpy(h["w"]).to(dev)
    L, H, I = c["L"], c["H"], c["I"]
    local = int(((h["routes"] >= 0) & (h["routes"] < L)).sum())
    hi = H * I
    grads = {"dX": torch.empty_like(h["X"]),
             "dW13": torch.empty((L, 2 * I, H), dtype=torch.float32, device=dev),
             "dW2": torch.empty((L, H, I), dtype=torch.float32, device=dev),
             "dw": torch.empty((c["P"], c["Np"], c["K"]), dtype=torch.float32, device=dev)}

    def timed(step, steps):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ops.moe_trace_enable(steps * 64)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        per = {}
        for name, t in ops.moe_trace_read(steps * 64):
            per.setdefault(name, []).append(t)
        ops.moe_trace_enable(0)
        return e0.elapsed_time(e1) / steps, {k: float(np.sum(v)) / steps for k, v in per.items()}

    res = []
    # ring-less: fused dispatch for the forward alone; the backward needs the dispatched rows
    b = ops.alloc_fwd(d, dev, save_hu=True, save_xd=True)
    bf = ops.alloc_fwd(d, dev, save_hu=True, save_xd=False)
    ws = torch.empty(ops.workspace_bytes(d, ops.MOE_OP_LAYER_BWD), dtype=torch.uint8, device=dev)
    fwd_ms, fwd_st = timed(lambda: ops.layer_fwd(d, routes, w, h["X"], h["W13"], h["W2"], bf), args.steps)

    def std_step():
        ops.layer_fwd(d, routes, w, h["X"], h["W13"], h["W2"], b)
        ops.moe_layer_bwd(d, h["dOut"], routes, w, b.phi, b.route_row, b.seg_off, b.Xd, b.HU, b.A, h["W13"],
                          h["W2"], grads["dX"], grads["dW13"], grads["dW2"], grads["dw"], ws)

    fb_ms, _ = timed(std_step, max(2, args.steps // 2))
    cap = ops.capacity_rows(d)
    res.append({"mb_tokens": c["Np"], "slots": None, "macrobatches": 1, "fwd_ms": fwd_ms, "fwd_bwd_ms": fb_ms,
                "dispatched_rows": int(b.seg_off[-1].item()), "replays": 0,
                "row_buffer_gb": cap * (H + 2 * I + I + H) * 2 / 1e9, "fwd_stage_ms": fwd_st})
    del b, bf, ws
    torch.cuda.empty_cache()
    for item in args.ring.split(","):
        B, S, G = (int(x) for x in (item.split(":") + ["1"])[:3])
        M = c["Np"] // B
        print(f"[bench] ring, {M} macrobatches of {B} tokens per partition, {S} slots, weight gradients in groups "
              f"of {G}", file=sys.stderr, flush=True)
        r = ops.alloc_ring(d, B, S, dev)
        ws = torch.empty(ops.ring_workspace_bytes(d, B, ops.MOE_OP_LAYER_BWD, G), dtype=torch.uint8, device=dev)
        fwd_ms, fwd_st = timed(lambda: ops.layer_fwd_ring(d, routes, w, h["X"], h["W13"], h["W2"], r), args.steps)

        def ring_step():
            ops.layer_fwd_ring(d, routes, w, h["X"], h["W13"], h["W2"], r)
            ops.moe_layer_bwd_ring(d, B, S, h["dOut"], w, h["X"], h["W13"], h["W2"], r.phi, r.route_row, r.seg_off,
                                   r.HU, r.A, grads["dX"], grads["dW13"], grads["dW2"], grads["dw"], ws, wgrad_group=G)

        fb_ms, fb_st = timed(ring_step, max(2, args.steps // 2))
        capm = ops.ring_capacity_rows(d, B)
        res.append({"mb_tokens": B, "slots": S, "wgrad_group": G, "macrobatches": M, "fwd_ms": fwd_ms, "fwd_bwd_ms": fb_ms,
                    "dispatched_rows": int(r.seg_off[:, -1].sum().item()), "replays": max(0, M - S),
                    "row_buffer_gb": (S * capm * 3 * I + capm * H) * 2 / 1e9, "fwd_stage_ms": fwd_st,
                    "replay_gateup_ms": fb_st.get("ring_replay_gateup", 0.0)})
        del r, ws
        torch.cuda.empty_cache()
    head = res[1] if len(res) > 1 else res[0]
    for x in res:
        x["fwd_tflops"] = 6.0 * hi * local / (x["fwd_ms"] / 1e3) / 1e12
        x["fwd_bwd_tflops"] = 18.0 * hi * local / (x["fwd_bwd_ms"] / 1e3) / 1e12
    return {"metric": "MoE layer fwd TFLOP/s through the macrobatch ring (Kimi shape, 1 GPU)",
            "value": head["fwd_tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": head["fwd_ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "kimi_local_share_ring", "P": c["P"], "tokens_per_partition": c["Np"],
                       "experts": c["E"], "local_experts": L, "top_k": c["K"], "H": H, "I": I,
                       "routing": "balanced", "local_routes": local, "mb_tokens": head["mb_tokens"],
                       "ring_slots": head["slots"]},
            "sweep": res}


def bench_shared(args, torch, ops, inputs, dev):
    """Kimi-shaped forward share with a shared expert (Is = --shared-is):
    moe_layer_fwd_shared (shared tiles inside the routed GEMM launches, the
    shared output added by the combine) beside the same work in separate
    launches (the routed forward, the shared expert as its own grouped GEMM,
    then an elementwise add)."""
    c = KIMI
    Is = args.shared_is
    h = inputs.make_layer_inputs_device(5, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], dev,
                                        routing="balanced", x_std=1.0)
    W13s = inputs.normal_bf16_device((2 * Is, c["H"]), 0.02, 91, dev)
    W2s = inputs.normal_bf16_device((c["H"], Is), 0.02, 92, dev)
    d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], c["L"], H=c["H"], I=c["I"])
    routes = torch.from_numpy(h["routes"]).to(dev)
    w = torch.from_numpy(h["w"]).to(dev)
    ntok = c["P"] * c["Np"]
    assert ntok % 256 == 0
    local = int(((h["routes"] >= 0) & (h["routes"] < c["L"])).sum())
    b = ops.alloc_fwd(d, dev, save_hu=True, save_xd=False)
    sh = ops.alloc_shared(d, Is, dev)
    ds = ops.make_desc(1, ntok, 1, 1, 1, H=c["H"], I=Is)
    seg_s = torch.tensor([0, ntok], dtype=torch.int32, device=dev)
    Xrows = h["X"].view(ntok, c["H"])
    ws_s = torch.empty(max(ops.workspace_bytes(ds, ops.MOE_OP_EXPERT_FFN), 256), dtype=torch.uint8, device=dev)

    def timed(step):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ops.moe_trace_enable(args.steps * 16)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        per = {}
        for name, t in ops.moe_trace_read(args.steps * 16):
            per.setdefault(name, []).append(t)
        ops.moe_trace_enable(0)
        return e0.elapsed_time(e1) / args.steps, {k: float(np.mean(v)) for k, v in per.items()}

    ms_f, st_f = timed(lambda: ops.layer_fwd_shared(d, routes, w, h["X"], h["W13"], h["W2"], W13s, W2s, b, sh))

    def separate():
        ops.layer_fwd(d, routes, w, h["X"], h["W13"], h["W2"], b)
        ops.moe_expert_ffn(ds, Xrows, W13s, W2s, seg_s, None, sh.As, sh.Ys, 0, ws_s)
        b.out.view(ntok, c["H"]).add_(sh.Ys[:ntok])

    ms_s, st_s = timed(separate)
    fl = 6.0 * c["H"] * c["I"] * local + 6.0 * c["H"] * Is * ntok
    return {"metric": "MoE layer fwd TFLOP/s with a shared expert (Kimi shape, 1 GPU)",
            "value": fl / (ms_f / 1e3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_f, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "kimi_local_share_fwd_shared_expert", "P": c["P"],
                       "tokens_per_partition": c["Np"], "experts": c["E"], "local_experts": c["L"], "top_k": c["K"],
                       "H": c["H"], "I": c["I"], "shared_I": Is, "routing": "balanced", "local_routes": local},
            "stage_ms": st_f,
            "separate_launches": {"ms_per_step": ms_s, "tflops": fl / (ms_s / 1e3) / 1e12, "stage_ms": st_s}}


PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA (no sparsity)


def bench_layer_mx(args, torch, ops, inputs, dev):
    """Kimi-shaped forward share with MXFP8 routed experts (moe_layer_fwd_mx):
    schedule, X quantization, MX gate/up GEMM pulling rows through the table
    with SwiGLU + quantization of a in its epilogue, MX down GEMM, combine.
    The weights are quantized once, before the timed region (they do not
    change between forward steps)."""
    c = KIMI
    h = inputs.make_layer_inputs_device(5, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], dev,
                                        routing="balanced", x_std=1.0)
    d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], c["L"], H=c["H"], I=c["I"])
    routes = torch.from_numpy(h["routes"]).to(dev)
    w = torch.from_numpy(h["w"]).to(dev)
    W13q, W13s = ops.quantize_mx(h["W13"])
    W2q, W2s = ops.quantize_mx(h["W2"])
    del h["W13"], h["W2"]
    bufs = ops.alloc_fwd_mx(d, dev)
    local = int(((h["routes"] >= 0) & (h["routes"] < c["L"])).sum())

    def step():
        ops.layer_fwd_mx(d, routes, w, h["X"], W13q, W13s, W2q, W2s, bufs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ops.moe_trace_enable(args.steps * 16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per = {}
    for name, t in ops.moe_trace_read(args.steps * 16):
        per.setdefault(name, []).append(t)
    ops.moe_trace_enable(0)
    st = {k: float(np.mean(v)) for k, v in per.items()}
    hi = c["H"] * c["I"]
    fl = 6.0 * hi * local
    gu = 4.0 * hi * local / (st["mx_gateup"] / 1e3) / 1e12
    dn = 2.0 * hi * local / (st["mx_down"] / 1e3) / 1e12
    return {"metric": "MoE layer fwd TFLOP/s, MXFP8 routed experts (Kimi shape, 1 GPU)",
            "value": fl / (ms / 1e3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "mxfp8-e4m3 (fp32 accumulate), bf16 in/out", "data": "synthetic",
            "config": {"workload": "kimi_local_share_fwd_mxfp8", "P": c["P"], "tokens_per_partition": c["Np"],
                       "experts": c["E"], "local_experts": c["L"], "top_k": c["K"], "H": c["H"], "I": c["I"],
                       "routing": "balanced", "local_routes": local, "weights": "quantized once, outside the step"},
            "stage_ms": st,
            "roofline": {"bound": "mfma", "kernel": "mx_gateup", "achieved": gu, "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": gu / PEAK_FP8_TFLOPS, "traffic": None,
                         "algorithmic_flop_per_launch": 4.0 * hi * local, "avg_launch_ms": st["mx_gateup"]},
            "mx_down": {"achieved": dn, "frac": dn / PEAK_FP8_TFLOPS, "avg_launch_ms": st["mx_down"]}}


def timed_steps(args, torch, ops, step, ntrace=64):
    """ms per call of step() over args.steps calls after args.warmup, and the
    mean launch time of every traced kernel."""
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ops.moe_trace_enable(args.steps * ntrace)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per = {}
    for name, t in ops.moe_trace_read(args.steps * ntrace):
        per.setdefault(name, []).append(t)
    ops.moe_trace_enable(0)
    return ms, {k: float(np.mean(v)) for k, v in per.items()}


def bench_fwd_bwd_mx(args, torch, ops, inputs, dev):
    """Kimi-shaped forward + backward with MXFP8 routed experts
    (moe_layer_fwd_mx saving h and u, then moe_layer_bwd_mx), beside the bf16
    forward + backward on the same inputs in the same process.  Weights are
    quantized before the timed region, both row-wise (forward) and column-wise
    (backward), as a training step would after each weight update."""
    c = KIMI
    routing = args.bwd_routing
    h = inputs.make_layer_inputs_device(6, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], dev,
                                        routing=routing, x_std=1.0, s=1.5, with_grad=True)
    d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], c["L"], H=c["H"], I=c["I"])
    routes = torch.from_numpy(h["routes"]).to(dev)
    w = torch.from_numpy(h["w"]).to(dev)
    L, H, I = c["L"], c["H"], c["I"]
    local = int(((h["routes"] >= 0) & (h["routes"] < L)).sum())
    W13q, W13s = ops.quantize_mx(h["W13"])
    W2q, W2s = ops.quantize_mx(h["W2"])
    W13t, W2t = ops.quantize_mx_t(h["W13"]), ops.quantize_mx_t(h["W2"])
    fm = ops.alloc_fwd_mx(d, dev, save_hu=True)
    gm = ops.alloc_bwd_mx(d, dev)

    def fwd_mx():
        ops.layer_fwd_mx(d, routes, w, h["X"], W13q, W13s, W2q, W2s, fm)

    def bwd_mx():
        ops.layer_bwd_mx(d, h["dOut"], w, h["X"], fm, W13t, W2t, gm)

    ms_fm, st_fm = timed_steps(args, torch, ops, fwd_mx)
    ms_bm, st_bm = timed_steps(args, torch, ops, bwd_mx)
    del fm, gm
    torch.cuda.empty_cache()
    b = ops.alloc_fwd(d, dev, save_hu=True)
    dX = torch.empty_like(h["X"])
    dW13 = torch.empty((L, 2 * I, H), dtype=torch.float32, device=dev)
    dW2 = torch.empty((L, H, I), dtype=torch.float32, device=dev)
    dw = torch.empty((c["P"], c["Np"], c["K"]), dtype=torch.float32, device=dev)
    ws = torch.empty(ops.workspace_bytes(d, ops.MOE_OP_LAYER_BWD), dtype=torch.uint8, device=dev)

    def fwd_bf16():
        ops.layer_fwd(d, routes, w, h["X"], h["W13"], h["W2"], b)

    def bwd_bf16():
        ops.moe_layer_bwd(d, h["dOut"], routes, w, b.phi, b.route_row, b.seg_off, b.Xd, b.HU, b.A, h["W13"],
                          h["W2"], dX, dW13, dW2, dw, ws)

    ms_fb, _ = timed_steps(args, torch, ops, fwd_bf16)
    ms_bb, st_bb = timed_steps(args, torch, ops, bwd_bf16)
    hi = H * I
    ms = ms_fm + ms_bm
    fl = 18.0 * hi * local
    tf = lambda flop, key, st: flop / (st[key] / 1e3) / 1e12 if key in st else None
    return {"metric": f"MoE layer fwd+bwd TFLOP/s, MXFP8 routed experts (Kimi shape, "
                      f"{'adversarial' if routing == 'hot' else routing} routing, 1 GPU)",
            "value": fl / (ms / 1e3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "mxfp8-e4m3 (fp32 accumulate), bf16 in/out", "data": "synthetic",
            "config": {"workload": "kimi_local_share_fwd_bwd_mxfp8",
                       "routing": "zipf1.5+4hot" if routing == "hot" else routing, "local_routes": local,
                       "weights": "quantized row- and column-wise once, outside the step"},
            "ms": {"fwd_mx": ms_fm, "bwd_mx": ms_bm, "fwd_bf16": ms_fb, "bwd_bf16": ms_bb},
            "speedup_vs_bf16": {"fwd": ms_fb / ms_fm, "bwd": ms_bb / ms_bm, "fwd_bwd": (ms_fb + ms_bb) / ms},
            "stage_ms_fwd_mx": st_fm, "stage_ms_bwd_mx": st_bm, "stage_ms_bwd_bf16": st_bb,
            "kernel_tflops": {k: v for k, v in {
                "mx_bwd_down": tf(2.0 * hi * local, "mx_bwd_down", st_bm),
                "mx_bwd_gateup": tf(4.0 * hi * local, "mx_bwd_gateup", st_bm),
                "mx_bwd_wgrad_rdispatch": tf(6.0 * hi * local, "mx_bwd_wgrad_rdispatch", st_bm)}.items()}}


def bench_tc_sweep(args, torch, ops, inputs, dev):
    """Mid configuration (8 x 4096 tokens, 64 experts with 8 local, top-6, H=2048,
    I=1024): layer forward vs the minibatch of dispatched rows Tc (persistent
    launch, gate/up of chunk c overlapping the down projection of chunk c-1)."""
    P, Np, E, K, L, H, I = 8, 4096, 64, 6, 8, 2048, 1024
    h = inputs.make_layer_inputs_device(4, P, Np, E, K, L, H, I, dev, routing="uniform", x_std=1.0)
    d = ops.make_desc(P, Np, K, E, L, H=H, I=I)
    routes = torch.from_numpy(h["routes"]).to(dev)
    w = torch.from_numpy(h["w"]).to(dev)
    b = ops.alloc_fwd(d, dev, save_hu=False)
    local = int(((h["routes"] >= 0) & (h["routes"] < L)).sum())
    fl = 6.0 * H * I * local
    rows = []
    for label, flags, tc in [("multi-launch", 0, 0), ("persistent", ops.MOE_PERSISTENT, 0)] + \
            [("persistent", ops.MOE_PERSISTENT, t) for t in (256, 512, 1024, 2048, 4096, 8192)]:
        for _ in range(args.warmup):
            ops.layer_fwd(d, routes, w, h["X"], h["W13"], h["W2"], b, flags=flags, chunk_rows=tc)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            ops.layer_fwd(d, routes, w, h["X"], h["W13"], h["W2"], b, flags=flags, chunk_rows=tc)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        rows.append({"path": label, "chunk_rows": tc, "ms": ms, "tflops": fl / (ms / 1e3) / 1e12})
    npad = int(b.seg_off[-1].item())
    return {"metric": "MoE layer fwd ms vs minibatch Tc (mid shape, 1 GPU)", "unit": "ms",
            "config": {"workload": "mid_fwd_tc_sweep", "P": P, "tokens_per_partition": Np, "experts": E,
                       "local_experts": L, "top_k": K, "H": H, "I": I, "local_routes": local,
                       "dispatched_rows": npad,
                       "tc_floor_cdna4_256x256": 2 * 256 * 256 * 256 // min(2 * I, H)},
            "sweep": rows}


def bench_vendor_gemm(args, torch, ops, inputs, dev):
    """Context for the grouped GEMMs: the vendor BLAS (torch -> hipBLASLt) on
    the same shapes in the same process, next to this library's gate/up and
    down launches of the Kimi-shaped layer forward.  The vendor products are
    plain GEMMs (no SwiGLU, no gather, no HU copy), so they bound from above
    what a library GEMM of these shapes reaches on this machine:
      batched_nn     48 experts x 1,280 rows: X[l] (1280 x 7168) @ W[l] (7168 x 4096),
                     one weight per expert, torch.bmm (weights stored K x N);
      per_expert_nt  the same, as 48 products X[l] @ W[l]^T with W[l] stored
                     4096 x 7168 (the layout of W13: both operands K-contiguous);
      dense_nt       61,440 x 7168 @ (4096 x 7168)^T, one weight for all rows;
      down_*         the down projection shapes (K = 2048, N = 7168)."""
    print("[bench] this library's layer forward", file=sys.stderr, flush=True)
    L_res = bench_layer(args, torch, ops, inputs, dev)
    st = L_res["stage_ms"]
    ours = {"ffn_gateup": {"ms": st["ffn_gateup"], "tflops": L_res["flops_gateup"] / st["ffn_gateup"] / 1e9},
            "ffn_down": {"ms": st["ffn_down"], "tflops": L_res["flops_down"] / st["ffn_down"] / 1e9}}
    del L_res
    torch.cuda.empty_cache()
    c = KIMI
    L, Mb, H, I = c["L"], 1280, c["H"], c["I"]
    g = torch.Generator(device=dev)
    g.manual_seed(7)

    def randn(*shape, std):
        return (torch.randn(*shape, device=dev, generator=g, dtype=torch.float32) * std).to(torch.bfloat16)

    def timed(fn, flops):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        return {"ms": ms, "tflops": flops / ms / 1e9}

    vendor = {}
    fl_gu = 2.0 * L * Mb * H * 2 * I
    fl_dn = 2.0 * L * Mb * I * H
    print("[bench] vendor gate/up shapes", file=sys.stderr, flush=True)
    Xb = randn(L, Mb, H, std=1.0)
    Wkn = randn(L, H, 2 * I, std=0.02)  # stored K x N: bmm takes it without a transposed view
    vendor["batched_nn"] = timed(lambda: torch.bmm(Xb, Wkn), fl_gu)
    del Wkn
    Wnk = randn(L, 2 * I, H, std=0.02)
    outs = torch.empty(L, Mb, 2 * I, device=dev, dtype=torch.bfloat16)

    def per_expert():
        for l in range(L):
            torch.matmul(Xb[l], Wnk[l].t(), out=outs[l])

    vendor["per_expert_nt"] = timed(per_expert, fl_gu)
    Xflat = Xb.view(L * Mb, H)
    vendor["dense_nt"] = timed(lambda: torch.matmul(Xflat, Wnk[0].t()), fl_gu)
    del Xb, Wnk, outs, Xflat
    torch.cuda.empty_cache()
    print("[bench] vendor down shapes", file=sys.stderr, flush=True)
    Ab = randn(L, Mb, I, std=1.0)
    W2kn = randn(L, I, H, std=0.02)
    vendor["down_batched_nn"] = timed(lambda: torch.bmm(Ab, W2kn), fl_dn)
    del W2kn
    W2nk = randn(L, H, I, std=0.02)
    outd = torch.empty(L, Mb, H, device=dev, dtype=torch.bfloat16)

    def per_expert_down():
        for l in range(L):
            torch.matmul(Ab[l], W2nk[l].t(), out=outd[l])

    vendor["down_per_expert_nt"] = timed(per_expert_down, fl_dn)
    return {"metric": "grouped GEMM TFLOP/s vs the vendor BLAS on the same shapes (Kimi share, 1 GPU)",
            "unit": "TFLOP/s", "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "kimi_gemm_vendor_context", "experts": L, "rows_per_expert": Mb, "H": H, "I": I},
            "this_library": ours, "vendor_blas": vendor,
            "torch": torch.__version__, "hip": torch.version.hip}


def cpu_baseline(L_res, torch, oracle, budget_s: float):
    """The oracle's per-token forward on a bounded sample of tokens."""
    c = KIMI
    h = L_res["h"]
    ntok = c["P"] * c["Np"]
    rng = np.random.default_rng(0)
    # host copies (bf16 bit patterns) of what the oracle reads
    X = h["X"].view(torch.int16).cpu().numpy().view(np.uint16)
    W13 = h["W13"].view(torch.int16).cpu().numpy().view(np.uint16)
    W2 = h["W2"].view(torch.int16).cpu().numpy().view(np.uint16)
    routes, w = h["routes"], h["w"]
    # calibrate on a few tokens, then size the sample to about budget_s seconds
    n = 16
    t0 = time.perf_counter()
    oracle.layer_fwd_tokens(routes, w, X, W13, W2, L=c["L"], tokens=rng.choice(ntok, n, replace=False))
    t1 = time.perf_counter() - t0
    n = int(min(ntok, max(32, n * budget_s / max(t1, 1e-3))))
    toks = np.sort(rng.choice(ntok, n, replace=False))
    t0 = time.perf_counter()
    oracle.layer_fwd_tokens(routes, w, X, W13, W2, L=c["L"], tokens=toks)
    dt = time.perf_counter() - t0
    local = int(((routes.reshape(-1, c["K"])[toks] >= 0) & (routes.reshape(-1, c["K"])[toks] < c["L"])).sum())
    flops = 6.0 * c["H"] * c["I"] * local
    # schedule oracle (serial plain definition) on one routing tensor
    t0 = time.perf_counter()
    oracle.schedule(routes, c["L"], 0, 256)
    ts = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"layer forward of {n} of {ntok} tokens ({local} local routes, 6*H*I flop each) "
                      f"in {dt:.1f} s, fp64 C with OpenMP",
            "schedule_routes_per_s": c["P"] * c["Np"] * c["K"] / ts,
            "schedule_sample": "one 458,752-route table, serial plain definition"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--persistent", action="store_true", help="time the persistent single-launch forward")
    ap.add_argument("--chunk-rows", type=int, default=0, help="minibatch of dispatched rows (multiple of 256)")
    ap.add_argument("--materialize-xd", action="store_true",
                    help="write the dispatched rows Xd with a separate gather (default: the gather is fused into the "
                         "gate/up GEMM's operand loads)")
    ap.add_argument("--sched-batches", type=int, default=64)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-schedule", action="store_true")
    ap.add_argument("--bwd-routing", default="hot", choices=["hot", "balanced"],
                    help="routing of --workload kimi_bwd (default: adversarial)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the layer steps, run one plain read+write kernel over this many MiB (counter scaling)")
    ap.add_argument("--workload", default="kimi",
                    choices=["kimi", "kimi_bwd", "mid_tc", "schedule", "kimi_mx", "kimi_mx_bwd", "kimi_ring",
                             "kimi_shared", "vendor_gemm"],
                    help="kimi: the contract line (default); kimi_bwd / mid_tc / schedule / kimi_mx / kimi_mx_bwd / "
                         "kimi_ring / kimi_shared: extra measurements; vendor_gemm: the vendor BLAS on the grouped "
                         "GEMMs' shapes, for context")
    ap.add_argument("--shared-is", type=int, default=2048, help="--workload kimi_shared: shared intermediate size")
    ap.add_argument("--ring", default="3584:1:1,3584:2:1,3584:2:2,1024:2:1,1024:2:7,1024:7:7",
                    help="--workload kimi_ring: comma list of tokens-per-partition-per-macrobatch:slots[:wgrad group]")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} (world size {world}) is not "
              "supported: this library has no multi-GPU path (nothing is sent between GPUs).", file=sys.stderr)
        sys.exit(2)

    import torch

    import oracle
    from routing_schedule_expert_amd import inputs, ops

    ops.load()
    dev = torch.device("cuda:0")
    if args.workload == "kimi_bwd":
        print(json.dumps(bench_fwd_bwd(args, torch, ops, inputs, dev)), flush=True)
        return
    if args.workload == "mid_tc":
        print(json.dumps(bench_tc_sweep(args, torch, ops, inputs, dev)), flush=True)
        return
    if args.workload == "kimi_mx_bwd":
        print(json.dumps(bench_fwd_bwd_mx(args, torch, ops, inputs, dev)), flush=True)
        return
    if args.workload == "kimi_mx":
        print(json.dumps(bench_layer_mx(args, torch, ops, inputs, dev)), flush=True)
        return
    if args.workload == "kimi_ring":
        print(json.dumps(bench_ring(args, torch, ops, inputs, dev)), flush=True)
        return
    if args.workload == "kimi_shared":
        print(json.dumps(bench_shared(args, torch, ops, inputs, dev)), flush=True)
        return
    if args.workload == "schedule":
        print(json.dumps(bench_schedule_sweep(args, torch, ops, inputs, dev)), flush=True)
        return
    if args.workload == "vendor_gemm":
        print(json.dumps(bench_vendor_gemm(args, torch, ops, inputs, dev)), flush=True)
        return
    print("[bench] layer forward, Kimi shape", file=sys.stderr, flush=True)
    L_res = bench_layer(args, torch, ops, inputs, dev)
    if args.copy_calibration_mib > 0:
        copy_calibration(torch, dev, args.copy_calibration_mib)
    ms = L_res["ms_step"]
    value = L_res["flops"] / (ms / 1e3) / 1e12
    st = L_res["stage_ms"]
    k_main = "ffn_gateup" if "ffn_gateup" in st else None
    roofline = None
    if k_main:
        ach = L_res["flops_gateup"] / (st[k_main] / 1e3) / 1e12
        roofline = {"bound": "mfma", "kernel": k_main, "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": ach / PEAK_BF16_TFLOPS, "traffic": measured_traffic(k_main),
                    "algorithmic_flop_per_launch": L_res["flops_gateup"], "avg_launch_ms": st[k_main]}
    down = None
    if "ffn_down" in st:
        ach = L_res["flops_down"] / (st["ffn_down"] / 1e3) / 1e12
        down = {"achieved": ach, "frac": ach / PEAK_BF16_TFLOPS, "avg_launch_ms": st["ffn_down"]}
    sched = None
    if not args.no_schedule:
        print("[bench] schedule only, 64 routing tensors per call", file=sys.stderr, flush=True)
        s64 = bench_schedule(args, torch, ops, inputs, dev, args.sched_batches)
        s1 = bench_schedule(args, torch, ops, inputs, dev, 1)
        sched = {"nb": s64["nb"], "routing": "uniform", "routes_per_s": s64["routes_per_s"], "ms": s64["ms"],
                 "kernel_ms": s64["split_ms"],
                 "achieved_GBs": s64["gbs"], "peak_GBs": PEAK_HBM_GBS, "frac": s64["hbm_frac"],
                 "compulsory_bytes_per_call": s64["compulsory_bytes"],
                 "nb1_ms": s1["ms"], "nb1_routes_per_s": s1["routes_per_s"],
                 "share_of_layer_nb1": s1["ms"] / ms}
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(L_res, torch, oracle, args.cpu_budget)
    c = KIMI
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kimi_local_share_fwd", "P": c["P"], "tokens_per_partition": c["Np"],
                   "experts": c["E"], "local_experts": c["L"], "top_k": c["K"], "H": c["H"], "I": c["I"],
                   "routing": "balanced", "pad_rows": 256, "dispatched_rows": L_res["npad"],
                   "local_routes": L_res["local_routes"], "path": "persistent" if args.persistent else "multi-launch",
                   "chunk_rows": args.chunk_rows,
                   "dispatch": "separate gather" if args.materialize_xd else "fused into the gate/up operand loads"},
        "mfma_util_from_time": value / PEAK_BF16_TFLOPS,
        "mfma_counters": measured_mfma_counters(),
        "stage_ms": st,
        "roofline": roofline,
        "ffn_down": down,
        "schedule": sched,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
