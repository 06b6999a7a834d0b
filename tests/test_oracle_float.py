"""Pins for the oracle's float path (CPU only).

  * dispatch is a bit copy by definition;
  * dense special case: every expert holds the same weights, every expert is
    local and each token's weights sum to one, so the layer output is the plain
    SwiGLU FFN of the token, computed here with torch fp64 matmuls;
  * K = 1 and w = 1 turn the combine into an un-permute of Y;
  * the schedule route (dispatch -> per-row FFN -> combine) and the direct
    per-token route agree;
  * backward: torch fp64 autograd of the same layer, central finite differences
    of the oracle's own forward, and the identity dw = <dOut, y>.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs


def f64(bits):
    return inputs.bf16_to_f32(bits).astype(np.float64)


def tiny(seed=1, P=2, Np=16, E=6, K=2, L=3, H=32, I=16, routing="topk", x_std=1.0):
    d = inputs.make_layer_inputs(seed, P, Np, E, K, L, H, I, routing=routing, x_std=x_std, with_grad=True)
    return d


def test_dispatch_is_bit_copy():
    d = tiny()
    s = oracle.schedule(d["routes"], 3, 0, 4)
    Xd = oracle.dispatch(d["X"], s.phi)
    for row in range(s.npad):
        part, tok = s.phi[row]
        if part < 0:
            assert not Xd[row].any()
        else:
            np.testing.assert_array_equal(Xd[row], d["X"][part, tok])


def test_dense_special_case_matches_torch():
    """Identical experts, all local, weights summing to one: out = SwiGLU_FFN(x)."""
    rng = inputs.rng_for(3)
    P, Np, E, K, H, I = 2, 24, 4, 3, 48, 40
    routes, w = inputs.routes_uniform(rng, P, Np, E, K)
    X = inputs.normal_bf16(rng, (P, Np, H), 1.0)
    W13one = inputs.normal_bf16(rng, (2 * I, H), 0.1)
    W2one = inputs.normal_bf16(rng, (H, I), 0.1)
    W13 = np.ascontiguousarray(np.broadcast_to(W13one, (E, 2 * I, H)))
    W2 = np.ascontiguousarray(np.broadcast_to(W2one, (E, H, I)))
    x = torch.from_numpy(f64(X).reshape(-1, H))
    w13 = torch.from_numpy(f64(W13one))
    w2 = torch.from_numpy(f64(W2one))
    ref = (torch.nn.functional.silu(x @ w13[:I].T) * (x @ w13[I:].T)) @ w2.T
    ref = ref * torch.from_numpy(w.astype(np.float64).sum(-1).reshape(-1, 1))
    out = oracle.layer_fwd_tokens(routes, w, X, W13, W2, L=E)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)
    # and through the schedule route
    s = oracle.schedule(routes, E, 0, 8)
    Xd = oracle.dispatch(X, s.phi)
    Y = oracle.expert_ffn_rows(s.seg_off, Xd, W13, W2, want=("Y",))["Y"]
    out2 = oracle.combine(s.route_row, w, Y)
    np.testing.assert_allclose(out2, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_k1_combine_is_unpermute():
    d = tiny(K=1, routing="uniform")
    w = np.ones_like(d["w"])
    s = oracle.schedule(d["routes"], 3, 0, 4)
    Xd = oracle.dispatch(d["X"], s.phi)
    Y = oracle.expert_ffn_rows(s.seg_off, Xd, d["W13"], d["W2"], want=("Y",))["Y"]
    out = oracle.combine(s.route_row, w, Y)
    rr = s.route_row.reshape(-1)
    for g in range(rr.size):
        if rr[g] < 0:
            assert not out[g].any()
        else:
            np.testing.assert_array_equal(out[g], Y[rr[g]])


def test_schedule_route_equals_token_route():
    for seed, L, base in ((4, 3, 0), (5, 2, 3), (6, 6, 0)):
        d = tiny(seed=seed, E=6, K=3, L=L, routing="uniform")
        W13, W2 = d["W13"], d["W2"]
        s = oracle.schedule(d["routes"], L, base, 4)
        Xd = oracle.dispatch(d["X"], s.phi)
        r = oracle.expert_ffn_rows(s.seg_off, Xd, W13, W2)
        out = oracle.combine(s.route_row, d["w"], r["Y"])
        ref = oracle.layer_fwd_tokens(d["routes"], d["w"], d["X"], W13, W2, L=L, base=base)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)
        # padding rows produce exactly zero
        pad_rows = s.phi[:, 0] < 0
        assert not r["Y"][pad_rows].any() and not r["A"][pad_rows].any()
        # row subset == full evaluation
        rows = np.array([0, s.npad - 1, s.npad // 2])
        sub = oracle.expert_ffn_rows(s.seg_off, Xd, W13, W2, rows=rows)
        np.testing.assert_array_equal(sub["Y"], r["Y"][rows])


def test_combine_linear_in_w():
    d = tiny(seed=8)
    s = oracle.schedule(d["routes"], 3, 0, 4)
    Y = oracle.expert_ffn_rows(s.seg_off, oracle.dispatch(d["X"], s.phi), d["W13"], d["W2"], want=("Y",))["Y"]
    a = oracle.combine(s.route_row, d["w"], Y)
    b = oracle.combine(s.route_row, 2 * d["w"], Y)
    np.testing.assert_allclose(b, 2 * a, rtol=1e-14)


def torch_layer(routes, w, X, W13, W2, L, base):
    """fp64 torch forward of the layer for autograd (per expert, vectorised)."""
    P, Np, K = routes.shape
    H = X.shape[-1]
    I = W13.shape[1] // 2
    x = torch.tensor(f64(X).reshape(-1, H), requires_grad=True)
    w13 = torch.tensor(f64(W13), requires_grad=True)
    w2 = torch.tensor(f64(W2), requires_grad=True)
    wt = torch.tensor(w.astype(np.float64).reshape(-1, K), requires_grad=True)
    out = torch.zeros(P * Np, H, dtype=torch.float64)
    flat = routes.reshape(-1, K)
    for l in range(L):
        g, j = np.nonzero(flat == base + l)
        if g.size == 0:
            continue
        gi, ji = torch.from_numpy(g), torch.from_numpy(j)
        xs = x[gi]
        a = torch.nn.functional.silu(xs @ w13[l, :I].T) * (xs @ w13[l, I:].T)
        y = a @ w2[l].T
        out = out.index_add(0, gi, wt[gi, ji].unsqueeze(1) * y)
    return out, (x, w13, w2, wt)


def test_backward_matches_torch_autograd():
    for seed, L, base, E, K in ((11, 3, 0, 6, 2), (12, 2, 1, 5, 3)):
        d = tiny(seed=seed, E=E, K=K, L=L, routing="uniform")
        g = oracle.layer_bwd(d["routes"], d["w"], d["X"], d["W13"], d["W2"], d["dOut"], L=L, base=base)
        out, (x, w13, w2, wt) = torch_layer(d["routes"], d["w"], d["X"], d["W13"], d["W2"], L, base)
        out.backward(torch.from_numpy(f64(d["dOut"]).reshape(out.shape)))
        H = d["X"].shape[-1]
        np.testing.assert_allclose(g["dX"].reshape(-1, H), x.grad.numpy(), rtol=1e-9, atol=1e-13)
        np.testing.assert_allclose(g["dW13"], w13.grad.numpy(), rtol=1e-9, atol=1e-13)
        np.testing.assert_allclose(g["dW2"], w2.grad.numpy(), rtol=1e-9, atol=1e-13)
        # slots of non-local experts have no gradient; local slots match autograd
        local = (d["routes"] >= base) & (d["routes"] < base + L)
        np.testing.assert_allclose(g["dw"][local], wt.grad.numpy().reshape(local.shape)[local], rtol=1e-9, atol=1e-13)
        assert not g["dw"][~local].any()
        # the sampled entry points agree with the full one
        toks = np.array([0, 5, d["X"].shape[1] + 3])
        dX, dw = oracle.bwd_tokens(d["routes"], d["w"], d["X"], d["W13"], d["W2"], d["dOut"], L, base, toks)
        np.testing.assert_allclose(dX, g["dX"].reshape(-1, H)[toks], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(dw, g["dw"].reshape(-1, K)[toks], rtol=1e-12, atol=1e-15)
        I = d["W13"].shape[1] // 2
        e13 = [(0, 0), (I + 1, 3), (2 * I - 1, H - 1)]
        e2 = [(0, 0), (H - 1, I - 1), (5, 2)]
        for l in range(L):
            g13, g2 = oracle.wgrad_elems(d["routes"], d["w"], d["X"], d["W13"], d["W2"], d["dOut"], L, base, l, e13, e2)
            np.testing.assert_allclose(g13, [g["dW13"][l][n, k] for n, k in e13], rtol=1e-10, atol=1e-14)
            np.testing.assert_allclose(g2, [g["dW2"][l][m, n] for m, n in e2], rtol=1e-10, atol=1e-14)
            # the absolute-term sums bound the results, and the same call returns the same sums
            h13, h2, a13, a2 = oracle.wgrad_elems(d["routes"], d["w"], d["X"], d["W13"], d["W2"], d["dOut"], L, base,
                                                  l, e13, e2, with_abs=True)
            assert np.array_equal(h13, g13) and np.array_equal(h2, g2)
            assert np.all(a13 >= np.abs(g13) * (1 - 1e-12)) and np.all(a2 >= np.abs(g2) * (1 - 1e-12))


def _loss(d, X=None, W13=None, W2=None, w=None, L=3, base=0):
    out = oracle.layer_fwd_tokens(d["routes"], d["w"] if w is None else w, d["X"] if X is None else X,
                                  d["W13"] if W13 is None else W13, d["W2"] if W2 is None else W2, L=L, base=base)
    return float((out * f64(d["dOut"]).reshape(out.shape)).sum())


def _bf16_neighbours(bits):
    """bf16 bit patterns one ulp below and above, inside the same binade."""
    b = int(bits)
    mant = b & 0x7F
    assert 0 < mant < 0x7F
    return np.uint16(b - 1), np.uint16(b + 1)


def test_backward_central_differences():
    """Central differences of the oracle's forward (one bf16 ulp each way)."""
    d = tiny(seed=21, E=6, K=2, L=3, routing="uniform")
    g = oracle.layer_bwd(d["routes"], d["w"], d["X"], d["W13"], d["W2"], d["dOut"], L=3, base=0)
    rng = np.random.default_rng(0)
    checks = 0
    for name, grad in (("X", g["dX"]), ("W13", g["dW13"]), ("W2", g["dW2"])):
        arr = d[name]
        for _ in range(40):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            if not (0 < (int(arr[idx]) & 0x7F) < 0x7F) or (int(arr[idx]) & 0x7F80) == 0:
                continue
            lo, hi = _bf16_neighbours(arr[idx])
            a_lo, a_hi = arr.copy(), arr.copy()
            a_lo[idx], a_hi[idx] = lo, hi
            step = float(f64(np.array([hi]))[0] - f64(np.array([lo]))[0])
            fd = (_loss(d, **{name: a_hi}) - _loss(d, **{name: a_lo})) / step
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])) + 1e-3 * abs(grad[idx]), (name, idx)
            checks += 1
    assert checks > 60
    # router weights: the output is linear in w, so the difference is exact
    for _ in range(10):
        idx = tuple(int(rng.integers(0, s)) for s in d["w"].shape)
        eps = np.float32(1e-2)
        wp, wm = d["w"].copy(), d["w"].copy()
        wp[idx] += eps
        wm[idx] -= eps
        step = float(np.float64(wp[idx]) - np.float64(wm[idx]))
        fd = (_loss(d, w=wp) - _loss(d, w=wm)) / step
        np.testing.assert_allclose(fd, g["dw"][idx], rtol=1e-8, atol=1e-14)


def test_dw_is_inner_product_with_expert_output():
    """dw[g][j] = <dOut[g], y> with y the expert output of that route."""
    d = tiny(seed=31, E=6, K=3, L=3, routing="uniform")
    g = oracle.layer_bwd(d["routes"], d["w"], d["X"], d["W13"], d["W2"], d["dOut"], L=3, base=0)
    s = oracle.schedule(d["routes"], 3, 0, 4)
    Y = oracle.expert_ffn_rows(s.seg_off, oracle.dispatch(d["X"], s.phi), d["W13"], d["W2"], want=("Y",))["Y"]
    dOut = f64(d["dOut"])
    P, Np, K = d["routes"].shape
    for r in range(P):
        for t in range(Np):
            for j in range(K):
                row = s.route_row[r, t, j]
                ref = 0.0 if row < 0 else float(dOut[r, t] @ Y[row])
                assert abs(g["dw"][r, t, j] - ref) <= 1e-10 * max(1e-12, abs(ref)) + 1e-15


def test_wgrad_abs_sums_single_route():
    """With a single route to an expert each element is one term, so its
    absolute-term sum is exactly its magnitude."""
    rng = np.random.default_rng(31)
    P, Np, K, E, L, H, I = 1, 3, 1, 4, 4, 16, 8
    d = inputs.make_layer_inputs(31, P, Np, E, K, L, H, I, routing="uniform", x_std=1.0, with_grad=True)
    routes = np.array([[[0], [1], [1]]], np.int32)
    e13 = [(int(rng.integers(0, 2 * I)), int(rng.integers(0, H))) for _ in range(6)]
    e2 = [(int(rng.integers(0, H)), int(rng.integers(0, I))) for _ in range(6)]
    g13, g2, a13, a2 = oracle.wgrad_elems(routes, d["w"], d["X"], d["W13"], d["W2"], d["dOut"], L, 0, 0, e13, e2,
                                          with_abs=True)
    np.testing.assert_array_equal(a13, np.abs(g13))
    np.testing.assert_array_equal(a2, np.abs(g2))
