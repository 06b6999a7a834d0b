"""Pins for the oracle's schedule (CPU only).

The oracle's plain definition (position formula) is checked against things
that do not share its arithmetic:
  * a hand-derived worked example (tests/golden/schedule_worked_example.json);
  * a pure-Python brute force that builds per-(expert, partition) token lists
    in scan order and merges them round-robin, on 945 random tiny cases (the
    count of randomized CPU-reference cases in 'Scan once, scatter once') and
    exhaustively over every routing tensor of a few tiny shapes;
  * numpy's stable argsort (one partition: the schedule is a stable sort);
  * the closed form p = o*P + r when every partition sends the same count;
  * the printed route-read and counter counts at 384 experts, EP8, 7,168
    tokens, top-8 ('Scan once, scatter once');
  * structural invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from routing_schedule_expert_amd import inputs


def brute_force(routes, L, base, pad):
    """Round-robin merge of per-(expert, partition) lists; no position formula."""
    P, Np, K = routes.shape
    lists = [[[] for _ in range(P)] for _ in range(L)]
    for r in range(P):
        for t in range(Np):
            for j in range(K):
                e = int(routes[r, t, j])
                if base <= e < base + L:
                    lists[e - base][r].append((t, j))
    phi, seg_off = [], [0]
    route_row = -np.ones((P, Np, K), np.int64)
    counts = np.zeros((L, P), np.int64)
    for l in range(L):
        for r in range(P):
            counts[l, r] = len(lists[l][r])
        longest = max((len(x) for x in lists[l]), default=0)
        for o in range(longest):
            for r in range(P):
                if o < len(lists[l][r]):
                    t, j = lists[l][r][o]
                    route_row[r, t, j] = len(phi)
                    phi.append((r, t))
        while len(phi) % pad:
            phi.append((-1, -1))
        seg_off.append(len(phi))
    return counts, np.array(seg_off), np.array(phi, dtype=np.int64).reshape(-1, 2), route_row


def assert_same(s, ref):
    counts, seg_off, phi, route_row = ref
    np.testing.assert_array_equal(s.counts, counts)
    np.testing.assert_array_equal(s.seg_off, seg_off)
    np.testing.assert_array_equal(s.phi, phi)
    np.testing.assert_array_equal(s.route_row, route_row)
    assert s.npad == seg_off[-1]


def check_invariants(s, routes, L, base, pad):
    P, Np, K = routes.shape
    seg = s.seg_off
    local = (routes >= base) & (routes < base + L)
    # counts are the per-(expert, partition) histograms
    for r in range(P):
        h = np.bincount(routes[r][local[r]] - base, minlength=L)
        np.testing.assert_array_equal(s.counts[:, r], h)
    totals = s.counts.sum(axis=1)
    padded = (totals + pad - 1) // pad * pad
    np.testing.assert_array_equal(seg, np.concatenate([[0], np.cumsum(padded)]))
    assert np.all(np.diff(seg) % pad == 0)
    # every local route placed exactly once, and Phi inverts route_row
    rr = s.route_row
    assert np.all(rr[~local] == -1)
    rows = rr[local]
    assert rows.size == np.unique(rows).size
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < s.npad)
    for (r, t, j) in zip(*np.nonzero(local)):
        row = rr[r, t, j]
        assert tuple(s.phi[row]) == (r, t)
        l = routes[r, t, j] - base
        assert seg[l] <= row < seg[l] + totals[l]  # real rows first, padding at the tail
    # padding rows are exactly the rows no route reaches
    reached = np.zeros(s.npad, bool)
    reached[rows] = True
    assert np.all(s.phi[~reached] == -1)
    assert reached.sum() == totals.sum()
    # per-(expert, partition) tokens in ascending order of flat route index
    for l in range(L):
        for r in range(P):
            idx = [(t * K + j, rr[r, t, j]) for t in range(Np) for j in range(K) if routes[r, t, j] == base + l]
            got = [row for _, row in sorted(idx)]
            assert got == sorted(got)


def test_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "schedule_worked_example.json")))
    routes = np.array(g["routes"], np.int32)
    ref = (np.array(g["counts"]), np.array(g["seg_off"]), np.array(g["phi"]), np.array(g["route_row"]))
    for fn in (oracle.schedule, oracle.schedule_rescan):
        assert_same(fn(routes, g["L"], g["base"], g["pad"]), ref)
    for nt in (1, 2, 3, 1024):
        assert_same(oracle.schedule_counting(routes, g["L"], g["base"], g["pad"], NT=nt), ref)
    assert_same(oracle.schedule(routes, g["L"], g["base"], g["pad"]), brute_force(routes, g["L"], g["base"], g["pad"]))


def _random_case(rng):
    P = int(rng.integers(1, 6))
    Np = int(rng.integers(1, 9))
    K = int(rng.integers(1, 5))
    E = int(rng.integers(1, 13))
    L = int(rng.integers(1, E + 1))
    base = int(rng.integers(0, E - L + 1))
    pad = int(rng.choice([1, 2, 3, 4, 8]))
    # ids in [-1, E]: repeats, dropped (-1) and out-of-range ids all occur
    routes = rng.integers(-1, E + 1, size=(P, Np, K)).astype(np.int32)
    return routes, L, base, pad


def test_bruteforce_945_random():
    rng = np.random.default_rng(945)
    for _ in range(945):
        routes, L, base, pad = _random_case(rng)
        ref = brute_force(routes, L, base, pad)
        assert_same(oracle.schedule(routes, L, base, pad), ref)
        assert_same(oracle.schedule_rescan(routes, L, base, pad), ref)
        nt = int(rng.integers(1, 40))
        assert_same(oracle.schedule_counting(routes, L, base, pad, NT=nt), ref)


@pytest.mark.parametrize("P,Np,K,E,L,base,pad", [
    (2, 2, 2, 3, 2, 0, 2),
    (2, 2, 2, 3, 2, 1, 4),
    (2, 1, 2, 4, 2, 1, 2),
    (3, 1, 2, 3, 3, 0, 1),
])
def test_bruteforce_exhaustive(P, Np, K, E, L, base, pad):
    n = P * Np * K
    for ids in itertools.product(range(E), repeat=n):
        routes = np.array(ids, np.int32).reshape(P, Np, K)
        ref = brute_force(routes, L, base, pad)
        assert_same(oracle.schedule(routes, L, base, pad), ref)


def test_invariants_random():
    rng = np.random.default_rng(7)
    for _ in range(60):
        routes, L, base, pad = _random_case(rng)
        check_invariants(oracle.schedule(routes, L, base, pad), routes, L, base, pad)


def test_one_partition_is_stable_argsort():
    rng = np.random.default_rng(11)
    for _ in range(50):
        Np, K, L = int(rng.integers(1, 40)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
        pad = int(rng.choice([1, 4, 16]))
        routes = rng.integers(-1, L + 2, size=(1, Np, K)).astype(np.int32)
        s = oracle.schedule(routes, L, 0, pad)
        flat = routes.reshape(-1)
        local = np.nonzero((flat >= 0) & (flat < L))[0]
        order = local[np.argsort(flat[local], kind="stable")]
        # real rows of the table, read in segment order, are the stable sort
        real = s.phi[s.phi[:, 0] >= 0]
        np.testing.assert_array_equal(real[:, 1], order // K)
        assert np.all(real[:, 0] == 0)


def test_equal_counts_closed_form():
    """All M[l][r] equal to m: position p = o*P + r."""
    rng = np.random.default_rng(5)
    P, L, m = 4, 3, 5
    Np, K = L * m, 1
    routes = np.zeros((P, Np, K), np.int32)
    for r in range(P):
        routes[r, :, 0] = rng.permutation(np.repeat(np.arange(L), m))
    s = oracle.schedule(routes, L, 0, 8)
    for r in range(P):
        seen = np.zeros(L, int)
        for t in range(Np):
            l = routes[r, t, 0]
            o = seen[l]
            seen[l] += 1
            assert s.route_row[r, t, 0] == s.seg_off[l] + o * P + r


def test_printed_counts_at_kimi_shape(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "printed_counts.json")))
    P, Np, K, E = g["P"], g["Np"], g["K"], g["E"]
    L = E // P
    routes, _ = inputs.routes_uniform(inputs.rng_for(2), P, Np, E, K)
    s_new = oracle.schedule_counting(routes, L, 0, 256, NT=g["NT"])
    assert s_new.stats["route_reads"] == g["new_route_reads"]
    assert s_new.stats["counters"] == g["counters"]
    s_plain = oracle.schedule(routes, L, 0, 256)
    assert s_plain.stats["route_reads"] == g["new_route_reads"]
    s_old = oracle.schedule_rescan(routes, L, 0, 256)
    assert s_old.stats["route_reads"] == g["old_route_reads"]
    for s in (s_new, s_old):
        np.testing.assert_array_equal(s.phi, s_plain.phi)
        np.testing.assert_array_equal(s.route_row, s_plain.route_row)
    assert int(g["old_route_reads"] / g["new_route_reads"]) == 48  # "a 48x cut" (48.5)


def test_balanced_kimi_segments():
    routes, _ = inputs.routes_balanced(inputs.rng_for(5), 8, 7168, 384, 8)
    s = oracle.schedule(routes, 48, 0, 256)
    totals = s.counts.sum(axis=1)
    assert set(totals.tolist()) <= {1194, 1195}
    assert s.npad == 61440


def test_minibatch_floor(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "minibatch_floor.json")))
    assert oracle.minibatch_floor(g["C"], g["bm"], g["bn"], g["H"], g["I"]) == g["T"]


def test_capacity_bound_is_reached():
    """Every route local and every segment one row past a multiple of pad."""
    P, Np, K, L, pad = 2, 5, 2, 4, 4
    routes = np.zeros((P, Np, K), np.int32)
    # 20 routes over 4 experts, 5 each: segments of 8 rows, bound 20 + 4*3 = 32
    routes.reshape(-1)[:] = np.repeat(np.arange(L), 5)
    s = oracle.schedule(routes, L, 0, pad)
    assert s.npad == 32 == oracle.capacity_rows(P, Np, K, L, pad)


def test_invalid_ids_brute_force():
    """The oracle's count of ids outside [0, E) equals a per-id Python count
    on random tiny tensors that mix valid, negative and too-large ids."""
    rng = np.random.default_rng(77)
    for _ in range(50):
        P, Np, K, E = (int(rng.integers(1, 4)), int(rng.integers(1, 20)), int(rng.integers(1, 4)),
                       int(rng.integers(1, 9)))
        routes = rng.integers(-3, E + 3, size=(P, Np, K)).astype(np.int32)
        want = sum(1 for e in routes.reshape(-1).tolist() if not (0 <= e < E))
        assert oracle.invalid_ids(routes, E) == want
    assert oracle.invalid_ids(np.zeros((2, 3, 2), np.int32), 1) == 0
    assert oracle.invalid_ids(np.full((1, 4, 2), -1, np.int32), 8) == 8
