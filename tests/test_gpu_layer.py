"""GPU forward/backward of the layer share vs the CPU oracle.

Integer and copy outputs (schedule, dispatched rows) must match bit for bit;
every real row of HU, A and Y, every token of out and dX, and every row of
dW13 and dW2 must be within rel-L2 1e-2 of the fp64 oracle's row (dw, a dot
product per slot, within 1e-2 of max(|ref|, rms)); the persistent, chunked and
multi-launch forward paths are each checked against the oracle and agree
bitwise; repeated runs must be bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs, ops
from tests.helpers import (assert_elems, assert_rows, bits, digest, dev, expected_single_route_table, f64, fused_y_rows,
                           on_dev_mask, rel_l2, up, up_bf16)

pytestmark = pytest.mark.gpu
TOL = 1e-2


class Layer:
    """Inputs on host (bit patterns) and device, plus the forward buffers."""

    def __init__(self, seed, P, Np, E, K, L, H, I, routing="uniform", base=0, x_std=1.0, s=1.2, grad=True):
        self.h = inputs.make_layer_inputs(seed, P, Np, E, K, L, H, I, routing=routing, base=base, x_std=x_std,
                                          s=s, with_grad=grad)
        self.P, self.Np, self.E, self.K, self.L, self.H, self.I, self.base = P, Np, E, K, L, H, I, base
        self.d = ops.make_desc(P, Np, K, E, L, expert_base=base, H=H, I=I)
        self.routes = up(self.h["routes"])
        self.w = up(self.h["w"])
        self.X = up_bf16(self.h["X"])
        self.W13 = up_bf16(self.h["W13"])
        self.W2 = up_bf16(self.h["W2"])
        self.dOut = up_bf16(self.h["dOut"]) if grad else None

    def fwd(self, flags=0, chunk_rows=0, save_hu=True, save_xd=True, ws_fill=None, y_fill=None):
        b = ops.alloc_fwd(self.d, dev(), save_hu=save_hu, save_xd=save_xd)
        if ws_fill is not None:  # what an earlier call could have left there
            b.ws.view(torch.int32).fill_(ws_fill)
        if y_fill is not None:
            b.Y.view(torch.int16).fill_(y_fill)
        ops.layer_fwd(self.d, self.routes, self.w, self.X, self.W13, self.W2, b, flags=flags, chunk_rows=chunk_rows)
        torch.cuda.synchronize()
        return b

    def bwd(self, b):
        d, L, H, I = self.d, self.L, self.H, self.I
        g = {
            "dX": torch.empty_like(self.X),
            "dW13": torch.empty((L, 2 * I, H), dtype=torch.float32, device=dev()),
            "dW2": torch.empty((L, H, I), dtype=torch.float32, device=dev()),
            "dw": torch.empty((self.P, self.Np, self.K), dtype=torch.float32, device=dev()),
        }
        ws = torch.empty(ops.workspace_bytes(d, ops.MOE_OP_LAYER_BWD), dtype=torch.uint8, device=dev())
        ops.moe_layer_bwd(d, self.dOut, self.routes, self.w, b.phi, b.route_row, b.seg_off, b.Xd, b.HU, b.A,
                          self.W13, self.W2, g["dX"], g["dW13"], g["dW2"], g["dw"], ws)
        torch.cuda.synchronize()
        return g

    def oracle_schedule(self):
        return oracle.schedule(self.h["routes"], self.L, self.base, 256)


def ws_word(lay: Layer, b: ops.FwdBuffers, field: int) -> int:
    return ops.read_ws_words(b.ws, ops.workspace_field(lay.d, ops.MOE_OP_LAYER_FWD, field))[0]


def y_rows(lay, s, flags=0, chunk_rows=0):
    """Rows of Y the forward writes: every row, except on the fused path
    (separate launches, no chunks), where the rows of single-route tokens go
    straight to out."""
    if flags & ops.MOE_PERSISTENT or chunk_rows > 0:
        return np.ones(s.npad, bool)
    return fused_y_rows(lay.h["routes"], lay.L, lay.base, s.phi)


def check_fwd_full(lay: Layer, b: ops.FwdBuffers, flags=0, chunk_rows=0):
    h = lay.h
    s = lay.oracle_schedule()
    np.testing.assert_array_equal(b.counts.cpu().numpy(), s.counts)
    np.testing.assert_array_equal(b.seg_off.cpu().numpy(), s.seg_off)
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    np.testing.assert_array_equal(b.route_row.cpu().numpy(), s.route_row)
    assert ws_word(lay, b, ops.MOE_WS_INVALID_IDS) == oracle.invalid_ids(h["routes"], lay.E)
    if flags & ops.MOE_PERSISTENT or chunk_rows > 0:
        assert ws_word(lay, b, ops.MOE_WS_BARRIER_STATUS) == 0, "a device-wide wait gave up"
    if b.Xd is not None:
        Xd = oracle.dispatch(h["X"], s.phi)
        np.testing.assert_array_equal(bits(b.Xd[: s.npad]), Xd)
    else:
        Xd = oracle.dispatch(h["X"], s.phi)
    r = oracle.expert_ffn_rows(s.seg_off, Xd, h["W13"], h["W2"])
    real = s.phi[:, 0] >= 0
    written = y_rows(lay, s, flags, chunk_rows)
    for name, t in (("HU", b.HU), ("A", b.A), ("Y", b.Y)):
        if t is not None:
            sel = real & written if name == "Y" else real
            if sel.any():  # selected on the device: unwritten rows of Y may hold any bits
                assert_rows(name, f64(t[: s.npad][on_dev_mask(sel)]), r[name][sel], TOL, np.nonzero(sel)[0])
            # padding rows are exactly zero in every row output
            assert not f64(t[: s.npad][on_dev_mask(~real)]).any(), f"{name}: a padding row is not zero"
    out = oracle.layer_fwd_tokens(h["routes"], h["w"], h["X"], h["W13"], h["W2"], L=lay.L, base=lay.base)
    got = f64(b.out).reshape(out.shape)
    # every token, including those with no local slot, which must be exactly zero
    assert_rows("out", got, out, TOL)
    none_local = ~((h["routes"] >= lay.base) & (h["routes"] < lay.base + lay.L)).any(-1).reshape(-1)
    assert not got[none_local].any()


@pytest.mark.parametrize("L,E", [(4, 8), (8, 8)])
def test_tiny_forward(L, E):
    print(f"[layer] tiny forward L={L}", flush=True)
    lay = Layer(1, 2, 256, E, 2, L, 256, 128, routing="topk", x_std=0.02)
    check_fwd_full(lay, lay.fwd())


def test_small_forward_multi_tile():
    print("[layer] small forward, several tiles and ragged segments", flush=True)
    lay = Layer(3, 4, 700, 12, 3, 6, 512, 256, routing="zipf", s=1.2)
    check_fwd_full(lay, lay.fwd())


def test_forward_large_experts():
    """Experts of 11 and 9 M tiles next to small ones: the gate/up tiles of an
    expert with more than 8 M tiles sweep the N tiles in groups of 4 aligned
    to its first tile, the last group short (3, then 1); every row, output
    and gradient against the oracle."""
    print("[layer] forward + backward, experts of 11 and 9 M tiles", flush=True)
    lay = Layer(12, 4, 700, 8, 2, 4, 256, 128, routing="uniform")
    rt = lay.h["routes"].copy()
    rt[:, :, 0] = 1                 # 2,800 rows: 11 tiles
    rt[:3, :, 1] = 2                # 2,100 rows: 9 tiles
    rt[3, :, 1] = np.where(rt[3, :, 1] < 3, 5, rt[3, :, 1])  # partition 3's second slot off experts 1 and 2
    lay.h["routes"] = rt
    lay.routes = up(rt)
    s = lay.oracle_schedule()
    assert list(np.diff(s.seg_off)[1:3] // 256) == [11, 9]
    b = lay.fwd()
    check_fwd_full(lay, b)
    check_bwd_full(lay, lay.bwd(b))


def local_route_counts(lay):
    r = lay.h["routes"].reshape(-1, lay.K).astype(np.int64)
    return ((r >= lay.base) & (r < lay.base + lay.L)).sum(axis=1)


def test_forward_paths_agree_bitwise():
    """The multi-launch forward (whose down epilogue writes the outputs of the
    tokens with one local route) against the persistent and chunked paths
    (whose combine writes every token), on tokens with 0, 1 and several local
    routes."""
    lay = Layer(4, 4, 900, 16, 4, 8, 512, 384, routing="uniform")
    n = local_route_counts(lay)
    assert (n == 0).any() and (n == 1).any() and (n >= 2).any()
    ref = lay.fwd()
    yw = on_dev_mask(y_rows(lay, lay.oracle_schedule()))
    outs = [ref]
    for flags, chunk in ((ops.MOE_PERSISTENT, 0), (0, 256), (ops.MOE_PERSISTENT, 512), (0, 1024)):
        print(f"[layer] forward flags={flags} chunk_rows={chunk}", flush=True)
        outs.append(lay.fwd(flags=flags, chunk_rows=chunk))
    npad = int(ref.seg_off[-1])
    for (flags, chunk), b in zip(((ops.MOE_PERSISTENT, 0), (0, 256), (ops.MOE_PERSISTENT, 512), (0, 1024)), outs[1:]):
        assert ws_word(lay, b, ops.MOE_WS_BARRIER_STATUS) == 0, (flags, chunk)
        assert digest(b.out) == digest(ref.out)
        assert digest(b.Y[:npad][yw], b.A[:npad], b.HU[:npad]) == digest(ref.Y[:npad][yw], ref.A[:npad],
                                                                          ref.HU[:npad])
        assert digest(b.phi[:npad], b.route_row, b.seg_off) == digest(ref.phi[:npad], ref.route_row, ref.seg_off)


def single_route_table(lay, b, npad):
    off = ops.workspace_field(lay.d, ops.MOE_OP_LAYER_FWD, ops.MOE_WS_SINGLE_ROUTE)
    assert off >= 0
    return np.array(ops.read_ws_words(b.ws, off, 2 * npad), np.int32).reshape(npad, 2)


@pytest.mark.parametrize("fill", [None, 0])
def test_single_route_table_bit_exact(fill):
    """The per-row table the down epilogue reads, bit for bit against the one
    computed on the host from the oracle's schedule: (token, weight bits) for
    rows of tokens with one local route, (-1, 0) for the others and padding;
    also over a workspace filled beforehand with words naming token 0."""
    lay = Layer(4, 4, 900, 16, 4, 8, 512, 384, routing="uniform")
    b = lay.fwd(ws_fill=fill)
    s = lay.oracle_schedule()
    ref = expected_single_route_table(lay.h["routes"], lay.h["w"], lay.L, lay.base, s.phi)
    assert (ref[:, 0] >= 0).any() and (ref[:, 0] < 0).any()
    np.testing.assert_array_equal(single_route_table(lay, b, s.npad), ref)


def test_single_route_tokens():
    """Every token with exactly one local route (top-1 routing): the
    multi-launch forward writes every routed token's output from the down
    GEMM's epilogue (one partly padded M tile per expert, two wide column
    tiles and a narrow one; tokens routed elsewhere stay 0 from the combine),
    leaves every real row of Y as it was and writes its padding rows, and
    must match the oracle and, bitwise, the persistent path."""
    lay = Layer(15, 3, 211, 6, 1, 4, 1024, 256, routing="uniform")
    n = local_route_counts(lay)
    assert (n == 1).any() and (n == 0).any() and n.max() == 1
    sentinel = 0x7FC1  # a bf16 NaN no product yields
    b = lay.fwd(y_fill=sentinel)
    check_fwd_full(lay, b)
    s = lay.oracle_schedule()
    real = s.phi[:, 0] >= 0
    y = bits(b.Y[: s.npad])
    assert (y[real] == sentinel).all() and (y[~real] == 0).all()
    p = lay.fwd(flags=ops.MOE_PERSISTENT)
    assert digest(p.out) == digest(b.out)


def test_many_slots_per_token():
    """K = 70 slots per token (more than one wave's lanes: the combine counts a
    token's local routes in two ballots) with 2 local experts of 80, so
    tokens have 0, 1 or 2 local routes: the multi-launch forward against the
    oracle and, bitwise, the persistent path."""
    lay = Layer(17, 2, 96, 80, 70, 2, 256, 128, routing="topk")
    n = local_route_counts(lay)
    assert (n == 0).any() and (n == 1).any() and (n == 2).any()
    b = lay.fwd()
    check_fwd_full(lay, b)
    p = lay.fwd(flags=ops.MOE_PERSISTENT)
    assert digest(p.out) == digest(b.out)


@pytest.mark.parametrize("fill", [0, 2, -5])
def test_stale_workspace(fill):
    """The forward must not depend on what the workspace held before the call:
    filled with int32 words that name routes of tokens 0 and 1 (0, K), or
    with a negative word, the multi-launch forward (whose down epilogue reads
    a per-row table kept there, padding rows included) still matches the
    oracle and, bitwise, the persistent path."""
    print(f"[layer] stale workspace words {fill}", flush=True)
    lay = Layer(16, 2, 300, 8, 2, 4, 256, 128, routing="uniform")
    ref = lay.fwd(flags=ops.MOE_PERSISTENT)
    assert int(ref.seg_off[-1]) > int((local_route_counts(lay)).sum())  # padding rows present
    b = lay.fwd(ws_fill=fill)
    assert digest(b.out) == digest(ref.out)
    if fill == 0:
        check_fwd_full(lay, b)


@pytest.mark.parametrize("flags,chunk,save_xd", [(ops.MOE_PERSISTENT, 0, True), (0, 256, True),
                                                (ops.MOE_PERSISTENT, 512, False), (0, 1024, False)])
def test_persistent_and_chunked_vs_oracle(flags, chunk, save_xd):
    """The persistent and chunked paths checked directly against the oracle
    (several M tiles, ragged segments, chunks that cut through segments), with
    the barrier status word 0 afterwards."""
    print(f"[layer] vs oracle: flags={flags} chunk_rows={chunk} save_xd={save_xd}", flush=True)
    lay = Layer(11, 4, 700, 12, 3, 6, 512, 256, routing="zipf", s=1.2)
    b = lay.fwd(flags=flags, chunk_rows=chunk, save_xd=save_xd)
    check_fwd_full(lay, b, flags, chunk)


def test_forward_fused_dispatch_bitwise():
    """Xd = NULL: the gate/up GEMM pulls its rows from X through phi; every
    output must be bitwise the one of the materialised dispatch, on the
    multi-launch, persistent and chunked paths."""
    lay = Layer(9, 4, 900, 16, 4, 8, 512, 384, routing="zipf", s=1.2)
    ref = lay.fwd()
    npad = int(ref.seg_off[-1])
    yw = on_dev_mask(y_rows(lay, lay.oracle_schedule()))
    for flags, chunk in ((0, 0), (ops.MOE_PERSISTENT, 0), (0, 512), (ops.MOE_PERSISTENT, 256)):
        print(f"[layer] fused dispatch flags={flags} chunk_rows={chunk}", flush=True)
        b = lay.fwd(flags=flags, chunk_rows=chunk, save_xd=False)
        assert b.Xd is None
        if flags or chunk:
            assert ws_word(lay, b, ops.MOE_WS_BARRIER_STATUS) == 0, (flags, chunk)
        assert digest(b.out) == digest(ref.out)
        assert digest(b.Y[:npad][yw], b.A[:npad], b.HU[:npad]) == digest(ref.Y[:npad][yw], ref.A[:npad],
                                                                          ref.HU[:npad])
        assert digest(b.phi[:npad], b.route_row, b.seg_off) == digest(ref.phi[:npad], ref.route_row, ref.seg_off)


def test_fused_dispatch_vs_oracle():
    lay = Layer(10, 2, 256, 8, 2, 4, 256, 128, routing="topk", x_std=0.02)
    b = lay.fwd(save_xd=False)
    h = lay.h
    s = lay.oracle_schedule()
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    r = oracle.expert_ffn_rows(s.seg_off, oracle.dispatch(h["X"], s.phi), h["W13"], h["W2"])
    real = s.phi[:, 0] >= 0
    assert_rows("A", f64(b.A[: s.npad])[real], r["A"][real], TOL, np.nonzero(real)[0])
    sel = real & y_rows(lay, s)
    assert_rows("Y", f64(b.Y[: s.npad][on_dev_mask(sel)]), r["Y"][sel], TOL, np.nonzero(sel)[0])
    assert not f64(b.Y[: s.npad][on_dev_mask(~real)]).any()  # padding rows read the zero row
    out = oracle.layer_fwd_tokens(h["routes"], h["w"], h["X"], h["W13"], h["W2"], L=lay.L)
    assert_rows("out", f64(b.out).reshape(out.shape), out, TOL)


def test_fused_dispatch_widest_rows():
    """H = 32768, the widest row the fused dispatch supports (padding rows
    read a static zero row of that many elements): bitwise the materialised
    path, padding rows zero, output vs the oracle."""
    print("[layer] fused dispatch, H = 32768", flush=True)
    lay = Layer(14, 2, 64, 8, 2, 4, 32768, 128, routing="topk", x_std=0.02, grad=False)
    a = lay.fwd(save_xd=True)
    b = lay.fwd(save_xd=False)
    s = lay.oracle_schedule()
    assert torch.equal(a.out, b.out)
    yw = on_dev_mask(y_rows(lay, s))
    assert torch.equal(a.Y[: s.npad][yw], b.Y[: s.npad][yw])
    real = s.phi[:, 0] >= 0
    assert (~real).any() and not f64(b.Y[: s.npad][on_dev_mask(~real)]).any()
    h = lay.h
    out = oracle.layer_fwd_tokens(h["routes"], h["w"], h["X"], h["W13"], h["W2"], L=lay.L)
    assert_rows("out (H=32768)", f64(b.out).reshape(out.shape), out, TOL)


def test_forward_without_saved_hu():
    lay = Layer(5, 2, 300, 8, 2, 4, 256, 128)
    a = lay.fwd(save_hu=True)
    b = lay.fwd(save_hu=False)
    assert digest(a.out) == digest(b.out)


def test_no_local_routes():
    lay = Layer(6, 2, 128, 8, 2, 4, 256, 128, base=4)
    lay.h["routes"][:] = np.where(lay.h["routes"] >= 4, lay.h["routes"] - 4, lay.h["routes"])
    lay.routes = up(lay.h["routes"])
    b = lay.fwd()
    assert int(b.seg_off[-1]) == 0
    assert not f64(b.out).any()


def check_bwd_full(lay: Layer, g):
    h = lay.h
    ref = oracle.layer_bwd(h["routes"], h["w"], h["X"], h["W13"], h["W2"], h["dOut"], L=lay.L, base=lay.base)
    H, I = lay.H, lay.I
    # dX per token; dW13 and dW2 per weight row (every expert); dw per slot
    assert_rows("dX", f64(g["dX"]).reshape(-1, H), ref["dX"].reshape(-1, H), TOL)
    assert_rows("dW13", f64(g["dW13"]).reshape(-1, H), ref["dW13"].reshape(-1, H), TOL)
    assert_rows("dW2", f64(g["dW2"]).reshape(-1, I), ref["dW2"].reshape(-1, I), TOL)
    local = (h["routes"] >= lay.base) & (h["routes"] < lay.base + lay.L)
    dw = f64(g["dw"]).reshape(ref["dw"].shape)
    assert_elems("dw", dw[local.reshape(ref["dw"].shape)], ref["dw"][local.reshape(ref["dw"].shape)], TOL)
    assert not f64(g["dw"])[~local].any()


def test_tiny_backward():
    print("[layer] tiny backward", flush=True)
    lay = Layer(1, 2, 256, 8, 2, 4, 256, 128, routing="topk", x_std=1.0)
    check_bwd_full(lay, lay.bwd(lay.fwd()))


def test_small_backward_skewed():
    print("[layer] small backward, skewed routing", flush=True)
    lay = Layer(7, 4, 600, 16, 4, 8, 512, 256, routing="zipf", s=1.5)
    check_bwd_full(lay, lay.bwd(lay.fwd()))


def test_repeat_runs_bitwise_identical():
    lay = Layer(8, 4, 800, 16, 4, 8, 512, 256, routing="zipf", s=1.2)
    hashes = set()
    yw = on_dev_mask(y_rows(lay, lay.oracle_schedule()))
    for _ in range(3):
        b = lay.fwd()
        g = lay.bwd(b)
        npad = int(b.seg_off[-1])
        hashes.add(digest(b.out, b.Y[:npad][yw], g["dX"], g["dW13"], g["dW2"], g["dw"]))
    assert len(hashes) == 1


def test_mid_forward_sampled():
    """Mid configuration: 8 x 4096 tokens, 64 experts (8 local), top-6, H=2048, I=1024."""
    print("[layer] mid forward (sampled rows and tokens)", flush=True)
    c = inputs.CONFIGS["mid"]
    lay = Layer(4, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], routing="uniform", grad=False)
    b = lay.fwd()
    s = lay.oracle_schedule()
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    np.testing.assert_array_equal(b.route_row.cpu().numpy(), s.route_row)
    Xd = oracle.dispatch(lay.h["X"], s.phi)
    np.testing.assert_array_equal(bits(b.Xd[: s.npad]), Xd)
    rng = np.random.default_rng(0)
    real = np.nonzero(s.phi[:, 0] >= 0)[0]
    rows = np.sort(rng.choice(real, 192, replace=False))
    r = oracle.expert_ffn_rows(s.seg_off, Xd, lay.h["W13"], lay.h["W2"], rows=rows)
    yw = y_rows(lay, s)[rows]
    assert yw.any() and (~yw).any()
    for name, t in (("HU", b.HU), ("A", b.A), ("Y", b.Y)):
        sel = yw if name == "Y" else np.ones(rows.size, bool)
        assert_rows(name, f64(t[rows[sel]]), r[name][sel], TOL, rows[sel])
    toks = np.sort(rng.choice(lay.P * lay.Np, 96, replace=False))
    out = oracle.layer_fwd_tokens(lay.h["routes"], lay.h["w"], lay.h["X"], lay.h["W13"], lay.h["W2"], L=lay.L,
                                  tokens=toks)
    assert_rows("out", f64(b.out).reshape(-1, lay.H)[toks], out, TOL, toks)


def test_random_shapes_forward_backward():
    """Seeded random shapes within the supported constraints (H a multiple of
    256, I of 128), routing kinds, expert bases and dropped slots: the full
    forward checks (tables bit-exact, rows and outputs vs the oracle, padding
    and non-local tokens exactly zero) and the full backward checks."""
    rng = np.random.default_rng(4242)
    for i in range(10):
        P = int(rng.integers(1, 5))
        Np = int(rng.integers(40, 500))
        E = int(rng.integers(4, 24))
        K = int(rng.integers(1, min(4, E) + 1))
        L = int(rng.integers(1, E + 1))
        base = int(rng.integers(0, E - L + 1))
        H = int(rng.choice([256, 512, 768]))
        I = int(rng.choice([128, 256, 384]))
        routing = str(rng.choice(["uniform", "zipf", "topk"]))
        drop = bool(rng.random() < 0.5)
        print(f"[layer] random {i}: P={P} Np={Np} E={E} K={K} L={L} base={base} H={H} I={I} {routing}"
              f"{' dropped slots' if drop else ''}", flush=True)
        lay = Layer(100 + i, P, Np, E, K, L, H, I, routing=routing, base=base, x_std=1.0)
        if drop:
            rt = lay.h["routes"].copy()
            rt[:, ::3, 0] = -1
            lay.h["routes"] = rt
            lay.routes = up(rt)
        b = lay.fwd()
        check_fwd_full(lay, b)
        check_bwd_full(lay, lay.bwd(b))
