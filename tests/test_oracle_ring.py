"""Pins of the macrobatch-ring bookkeeping in the oracle ("Beyond Peak TFLOPs"
section 2.B; Mixture-of-Kittens notes, section 4: a fixed ring of token
buffers, macrobatches cycling through it, the forward walking the ring in
reverse so that the backward's first macrobatches are still resident)."""
import numpy as np
import pytest

import oracle
from routing_schedule_expert_amd import inputs


def routes_of(seed, P, Np, E, K, routing="zipf"):
    return inputs.make_routes(routing, np.random.default_rng(seed), P, Np, E, K)[0]


def test_one_macrobatch_is_the_whole_table():
    r = routes_of(1, 3, 96, 16, 4)
    (one,) = oracle.macrobatch_schedules(r, 8, 96)
    full = oracle.schedule(r, 8)
    np.testing.assert_array_equal(one.phi, full.phi)
    np.testing.assert_array_equal(one.seg_off, full.seg_off)
    np.testing.assert_array_equal(one.route_row, full.route_row)


@pytest.mark.parametrize("B", [8, 24, 48])
def test_every_local_route_in_exactly_one_window(B):
    P, Np, E, K, L = 3, 96, 16, 4, 8
    r = routes_of(2, P, Np, E, K)
    tabs = oracle.macrobatch_schedules(r, L, B)
    full = oracle.schedule(r, L)
    assert len(tabs) == Np // B
    seen = np.zeros((P, Np, K), np.int32)
    for m, t in enumerate(tabs):
        # each window's table places its own routes: Phi rows point back at them
        for row, (p, tok) in enumerate(t.phi):
            if p < 0:
                continue
            js = np.nonzero(t.route_row[p, tok] == row)[0]
            assert len(js) == 1
            seen[p, m * B + tok, js[0]] += 1
        # the window's counts are the per-window split of the whole table's
        win = r[:, m * B:(m + 1) * B]
        for l in range(L):
            np.testing.assert_array_equal(t.counts[l], (win == l).sum(axis=(1, 2)))
        assert all(np.diff(t.seg_off) % 256 == 0)
    local = (r >= 0) & (r < L)
    np.testing.assert_array_equal(seen, local.astype(np.int32))
    assert sum(t.counts.sum() for t in tabs) == full.counts.sum()


@pytest.mark.parametrize("M,S", [(1, 1), (4, 1), (4, 2), (7, 3), (3, 5), (8, 8)])
def test_reversed_ring_residency_closed_form(M, S):
    walk, resident, replay = oracle.ring_walk(M, S)
    assert [m for m, _ in walk] == list(range(M - 1, -1, -1))
    # the last min(S, M) walked are the first min(S, M) macrobatches, each in slot (M-1-m) % S
    assert resident == {m: (M - 1 - m) % S for m in range(min(S, M))}
    assert replay == list(range(min(S, M), M))
    assert len(set(resident.values())) == len(resident)


@pytest.mark.parametrize("M,S", [(4, 1), (4, 2), (7, 3)])
def test_forward_order_walk_evicts_what_the_backward_needs_first(M, S):
    _, resident, replay = oracle.ring_walk(M, S, reverse=False)
    assert resident == {m: m % S for m in range(M - S, M)}
    assert replay[0] == 0 and len(replay) == M - S
    _, resident_r, _ = oracle.ring_walk(M, S)
    assert 0 in resident_r and 0 not in resident
